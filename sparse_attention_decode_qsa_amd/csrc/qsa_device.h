// qsa_device.h - shapes, vector types and wave/block helpers shared by the QSA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qsa {

// Compiled shapes.
constexpr int kPageSize = 64;                 // tokens per page
constexpr int kTokensPerBlock = 4;            // micro-block size (compression ratio 4)
constexpr int kBlocksPerPage = kPageSize / kTokensPerBlock;
constexpr int kIdxHeads = 4;
constexpr int kIdxDim = 64;
constexpr int kIdxTokenBytes = kIdxHeads * kIdxDim;          // 256
constexpr int kIdxPageBytes = kPageSize * kIdxTokenBytes;    // 16 KiB
constexpr int kHeadDim = 128;
constexpr int kMaxK = 512;                    // kept blocks
constexpr int kMaxGroup = 16;                 // query heads per KV head (MFMA rows)
constexpr int kMaxSlices = 64;
constexpr int kMaxQueries = 4096;             // new tokens per request in multi-token decode

// Host-side: byte counts of workspace regions are rounded up to 256.
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Context length of virtual request r = b*T + t when every request carries T draft tokens:
// draft token t sees L_b - (T-1-t) tokens, itself included (T = 1: request r itself, whose
// length 0 <= L_r is returned as it is). No branch, so loads issued next to it are not held
// behind it.
__device__ __forceinline__ int draft_length(const int32_t* lens, int r, int T) {
  const int b = r / T;
  return max(0, lens[b] - (T - 1 - (r - b * T)));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the row total.
__device__ __forceinline__ int row16_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false);  // row_ror:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false);  // row_ror:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false);  // row_ror:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false);  // row_ror:1
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave, all in DPP: a Hillis-Steele scan inside
// each 16-lane row (row_shr 1, 2, 4, 8; lanes shifted in from outside the row read 0), then
// row_bcast:15 adds row 0's total to row 1 and row 2's to row 3, and row_bcast:31 adds the
// total of rows 0-1 to rows 2-3.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Sum over the wave, returned in every lane (lane 63 of the inclusive scan).
__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane(wave_inclusive_scan((int)x), 63);
}

// Unsigned maximum over the wave, returned in every lane: the same DPP pattern with max,
// whose lane 63 sees every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, true));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t x) { return ~wave_max(~x); }

}  // namespace qsa
