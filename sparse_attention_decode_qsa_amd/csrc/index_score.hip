// index_score.hip - K1: int8 indexer scan, 4-token micro-block pooling, block scores.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: the indexer compresses keys into micro-blocks of 4 tokens and scores them.
// Block j of request b pools tokens 4j..4j+3 (those below L_b):
//     S[b][j] = sum_h sum_d q_idx[b][h][d] * sum_t key[t][h][d]
// The kernel forms the same integer by accumulating, token by token, int8 dot products
// against q_idx into the block's accumulator (sum_t dot(q, key_t) = dot(q, sum_t key_t)
// holds exactly in integer arithmetic), so the pooled key never has to be widened.
//
// Mapping. Grid (page groups, B): wave w of workgroup x scores page x*WAVES + w of
// request blockIdx.y (workgroups past the request's pages exit at once), one 16 KiB
// page = 16 blocks per wave:
//   lane = 16*r4 + c  (r4 = DPP row 0..3, c = 0..15)
//   load i (i = 0..15) of the lane reads the 16 bytes at offset 16*c of token
//   16*r4 + i of the page, so every load instruction reads four contiguous 256-byte
//   token rows. After 16 loads lane (r4, c) holds, for each of the blocks 4*r4 .. 4*r4+3,
//   the partial dot product of its 16 key bytes (head c/4, dims 16*(c%4)..+15) over the
//   block's 4 tokens. A 4-step DPP rotate-add inside each 16-lane row completes the sum
//   over the 256 key bytes of a token, and lanes c = 0..3 of row r4 store the scores of
//   blocks 4*r4 + c (64 contiguous bytes per page).
// Rows past L_b of the last page are read (the page is allocated) and masked to zero.
// Optionally the maximum block score of each page is written too (page_max[b][p]); the
// selection uses it to skip pages that cannot hold a kept block.
#include "qsa_device.h"

namespace qsa {

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void index_score_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages,
    int max_blocks, int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  const int b = blockIdx.y;
  const int L = lens[b];
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int p = blockIdx.x * WAVES + wave;
  if (p >= npages) return;
  const int r4 = lane >> 4, c = lane & 15;

  const int page = page_table[(size_t)b * max_pages + p];
  const i32x4 qv = *reinterpret_cast<const i32x4*>(q_idx + (size_t)b * kIdxTokenBytes + 16 * c);
  const int8_t* base = idx_cache + (size_t)page * kIdxPageBytes + r4 * (16 * kIdxTokenBytes) + 16 * c;

  i32x4 x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    x[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + i * kIdxTokenBytes));

  const int valid = L - p * kPageSize;  // tokens of this page below L (>= 1)
  if (valid < kPageSize) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (16 * r4 + i >= valid) x[i] = i32x4{0, 0, 0, 0};
  }

  int acc[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int a = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const i32x4 v = x[4 * r + t];
      a = __builtin_amdgcn_sdot4(v.x, qv.x, a, false);
      a = __builtin_amdgcn_sdot4(v.y, qv.y, a, false);
      a = __builtin_amdgcn_sdot4(v.z, qv.z, a, false);
      a = __builtin_amdgcn_sdot4(v.w, qv.w, a, false);
    }
    acc[r] = row16_sum(a);
  }

  const int nblk = (L + kTokensPerBlock - 1) / kTokensPerBlock;
  const int blk = p * kBlocksPerPage + 4 * r4 + c;
  if (c < 4 && blk < nblk) {
    const int v = c == 0 ? acc[0] : c == 1 ? acc[1] : c == 2 ? acc[2] : acc[3];
    scores[(size_t)b * max_blocks + blk] = v;
  }
  if (page_max) {
    const int first = p * kBlocksPerPage + 4 * r4;   // blocks of this DPP row
    int m = (int)0x80000000;
#pragma unroll
    for (int r = 0; r < 4; ++r) m = first + r < nblk ? max(m, acc[r]) : m;
    m = max(m, __shfl_xor(m, 16, 64));
    m = max(m, __shfl_xor(m, 32, 64));
    if (lane == 0) page_max[(size_t)b * max_pages + p] = m;
  }
}

constexpr int kScoreWaves = 16;

hipError_t launch_index_score(const int8_t* q_idx, const int8_t* idx_cache,
                              const int32_t* page_table, const int32_t* lens, int B,
                              int max_pages, int max_blocks, int32_t* scores, int32_t* page_max,
                              int num_cu, hipStream_t stream) {
  (void)num_cu;
  const unsigned gx = (unsigned)((max_pages + kScoreWaves - 1) / kScoreWaves);
  hipLaunchKernelGGL(index_score_kernel<kScoreWaves>, dim3(gx, B), dim3(kScoreWaves * 64), 0, stream,
                     q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max);
  return hipGetLastError();
}

}  // namespace qsa
