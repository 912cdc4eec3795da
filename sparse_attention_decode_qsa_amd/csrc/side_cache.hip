// side_cache.hip - the indexer's pooled-key side cache: build, decode-time append, and the
// indexer scan that reads it.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes": besides the main
// cache the indexer keeps a selector cache and side caches of its own (second paragraph), in the same cache
// group as the main cache, and synthetic batches must not write the side caches (bullets).
// Here the side cache holds the pooled key of every micro-block (the int sum of the int8
// keys of its up to 4 tokens, |sum| <= 512, stored as int16), page-aligned like the main
// cache: pooled[page][slot][4][64] with block j of a request in page page_table[j / 16],
// slot j % 16 (a 64-token page holds 16 blocks). A score read from it is the same integer
// as the scan over the int8 keys computes, from half the bytes (512 B per block instead of
// 4 x 256 B).
#include <hip/hip_ext.h>

#include "qsa_device.h"

namespace qsa {

void take_scan_events(hipEvent_t* start, hipEvent_t* stop);   // index_score.hip

constexpr int kSlotsPerPage = kPageSize / kTokensPerBlock;   // 16
constexpr int kPooledBlockBytes = kIdxTokenBytes * 2;        // 512
constexpr int kPooledPageBytes = kSlotsPerPage * kPooledBlockBytes;   // 8 KiB

__device__ __forceinline__ int sbyte(int w, int k) { return (int)(int8_t)(w >> (8 * k)); }

// ---------------------------------------------------------------------------------- build
// Grid (page groups, B), WAVES waves per workgroup, one page per wave. Lane = 16*r4 + c:
// load i reads the 16 key bytes at offset 16*c of token 16*r4 + i (as in the indexer scan),
// so after 16 loads the lane holds, for blocks 4*r4 + m (m = 0..3), the 16 keys of head c/4,
// dims 16*(c%4) .. +15 of its 4 tokens, and writes their int16 sums: 32 contiguous bytes of
// the block's 512. Tokens past L_b count as 0; blocks past ceil(L_b/4) are not written.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void pool_build_kernel(const int8_t* __restrict__ idx_cache,
                                                                const int32_t* __restrict__ page_table,
                                                                const int32_t* __restrict__ lens, int max_pages,
                                                                int16_t* __restrict__ pooled) {
  const int b = blockIdx.y, lane = lane_id(), wave = threadIdx.x >> 6;
  const int L = lens[b];
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int p = blockIdx.x * WAVES + wave;
  if (p >= npages) return;
  const int r4 = lane >> 4, c = lane & 15;
  const int page = page_table[(size_t)b * max_pages + p];
  const int valid = L - p * kPageSize;           // tokens of this page below L (>= 1)
  const int nblk = (L + kTokensPerBlock - 1) / kTokensPerBlock;
  const int8_t* base = idx_cache + (size_t)page * kIdxPageBytes + r4 * 16 * kIdxTokenBytes + 16 * c;
  i32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    v[i] = 16 * r4 + i < valid ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + i * kIdxTokenBytes))
                               : i32x4{0, 0, 0, 0};
  int8_t* out_page = reinterpret_cast<int8_t*>(pooled) + (size_t)page * kPooledPageBytes;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int blk = 4 * r4 + m;
    if (p * kSlotsPerPage + blk >= nblk) continue;
    int packed[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {       // dword w of the 16 bytes = keys 4w .. 4w+3
      int s[4] = {0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int x = v[4 * m + e][w];
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] += sbyte(x, k);
      }
      packed[2 * w] = (s[0] & 0xFFFF) | (s[1] << 16);
      packed[2 * w + 1] = (s[2] & 0xFFFF) | (s[3] << 16);
    }
    i32x4* dst = reinterpret_cast<i32x4*>(out_page + blk * kPooledBlockBytes + 32 * c);
    dst[0] = i32x4{packed[0], packed[1], packed[2], packed[3]};
    dst[1] = i32x4{packed[4], packed[5], packed[6], packed[7]};
  }
}

// --------------------------------------------------------------------------------- append
// One workgroup of 256 threads per request. The new token sits at t = L_b - 1: its K, V and
// indexer rows are copied into row t % 64 of page page_table[b][t / 64], and the side-cache
// entry of block t / 4 (same page, slot (t / 4) % 16) becomes the sum of the indexer rows
// of positions 4*(t/4) .. t, the last one taken from idx_new (it is not re-read from the
// cache). Thread i of 256 sums key element i. Requests with L_b = 0 or write[b] = 0 write
// nothing.
__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, const int8_t* __restrict__ idx_new,
    const int32_t* __restrict__ write, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    int8_t* __restrict__ idx_cache, int16_t* __restrict__ pooled, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ lens, int Hkv, int max_pages) {
  const int b = blockIdx.x, i = threadIdx.x;
  const int L = lens[b];
  if (L <= 0 || (write != nullptr && write[b] == 0)) return;
  const int t = L - 1;
  const int page = page_table[(size_t)b * max_pages + t / kPageSize];
  const int row = t % kPageSize;
  const size_t kv_row = ((size_t)page * kPageSize + row) * Hkv * kHeadDim;   // in bf16 elements
  const int nvec = Hkv * kHeadDim / 8;                                         // 16-byte vectors per row
  const i32x4* ks = reinterpret_cast<const i32x4*>(k_new + (size_t)b * Hkv * kHeadDim);
  const i32x4* vs = reinterpret_cast<const i32x4*>(v_new + (size_t)b * Hkv * kHeadDim);
  i32x4* kd = reinterpret_cast<i32x4*>(k_cache + kv_row);
  i32x4* vd = reinterpret_cast<i32x4*>(v_cache + kv_row);
  for (int x = i; x < nvec; x += 256) {
    kd[x] = ks[x];
    vd[x] = vs[x];
  }
  const int8_t* in = idx_new + (size_t)b * kIdxTokenBytes;
  int8_t* page_keys = idx_cache + (size_t)page * kIdxPageBytes;
  const int kin = in[i];
  page_keys[row * kIdxTokenBytes + i] = (int8_t)kin;
  if (pooled != nullptr) {
    const int first = row & ~(kTokensPerBlock - 1);
    int s = kin;
    for (int u = first; u < row; ++u) s += page_keys[u * kIdxTokenBytes + i];
    pooled[((size_t)page * kSlotsPerPage + row / kTokensPerBlock) * kIdxTokenBytes + i] = (int16_t)s;
  }
}

// ------------------------------------------------------------------------ scan of the side
// Grid (page groups, B), WAVES waves per workgroup, PPW consecutive 8 KiB side-cache pages
// (16 blocks each) per wave, all their loads issued first. Lane l = 32*hf + c: load i (i = 0..7) reads bytes [1024*i + 16*l, +16) of the page,
// i.e. int16 keys 8c .. 8c+7 (head c/8, dims 8*(c%8) .. +7) of block 2i + hf; the lane keeps
// the matching 8 query values as int16 pairs, so v_dot2 over its 4 dwords gives its part of
// the block's score and a sum over the 32 lanes of each half (DPP inside the 16-lane rows,
// then the partner row) completes it. Blocks past ceil(L_b/4) are neither written nor
// counted in the page maximum.
typedef short short2v __attribute__((ext_vector_type(2)));

// The decode step's cache writes, done by the scan (k_new == nullptr: none). The wave that
// scans the page holding the new token t = L_b - 1 writes its K/V/indexer rows and recomputes
// the side-cache entry of block t/4 from the block's earlier indexer rows plus the new key,
// and scores that block from the recomputed entry. Nothing else in the launch reads what it
// writes, so the results equal those of cache_append_kernel followed by the scan.
struct StepWrite {
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int8_t* idx_new;
  const int32_t* write;   // nullable: every request writes
  uint16_t* k_cache;
  uint16_t* v_cache;
  int8_t* idx_cache;
  int Hkv;
};

template <int WAVES, int PPW>
__global__ __launch_bounds__(WAVES * 64) void index_score_pooled_kernel(
    const int8_t* __restrict__ q_idx, int16_t* pooled, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ lens, int max_pages, int max_blocks, int32_t* __restrict__ scores,
    int32_t* __restrict__ page_max, StepWrite step) {
  const int b = blockIdx.y, lane = lane_id(), wave = threadIdx.x >> 6;
  const int p0 = (blockIdx.x * WAVES + wave) * PPW;   // the wave's PPW consecutive pages
  // The length and the wave's page-table entries (scalar loads at clamped indices, in bounds
  // whatever the length) are loaded together, and the empty asm keeps the entries ahead of
  // the exit test, so the keys wait for one round trip instead of two.
  const int L = lens[b];
  int pages[PPW];
#pragma unroll
  for (int k = 0; k < PPW; ++k)
    pages[k] = page_table[(size_t)b * max_pages + __builtin_amdgcn_readfirstlane(min(p0 + k, max_pages - 1))];
  asm volatile("" ::"s"(pages[0]));
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (p0 >= npages) return;
  const int hf = lane >> 5, c = lane & 31;
  const int nblk = (L + kTokensPerBlock - 1) / kTokensPerBlock;
  // query values 8c .. 8c+7 as int16 pairs
  const int2 qw = *reinterpret_cast<const int2*>(q_idx + (size_t)b * kIdxTokenBytes + 8 * c);
  short2v qd[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int w = e < 2 ? qw.x : qw.y;
    const int k0 = 2 * (e & 1);
    qd[e] = short2v{(short)sbyte(w, k0), (short)sbyte(w, k0 + 1)};
  }
  // every load of the wave's pages is issued before any arithmetic
  i32x4 v[PPW][8];
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    if (p0 + k >= npages) break;
    const int8_t* base = reinterpret_cast<const int8_t*>(pooled) + (size_t)pages[k] * kPooledPageBytes + 16 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[k][i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + 1024 * i));
  }
  const bool writes = step.k_new != nullptr && L > 0 && (step.write == nullptr || step.write[b] != 0);
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int p = p0 + k;
    if (p >= npages) break;
    if (writes && p == npages - 1) {   // this page holds the new token (the same for the whole wave)
      const int page = pages[k];
      const int row = (L - 1) % kPageSize;
      const size_t kv_row = ((size_t)page * kPageSize + row) * step.Hkv * kHeadDim;
      const int nvec = step.Hkv * kHeadDim / 8;
      const i32x4* ks = reinterpret_cast<const i32x4*>(step.k_new + (size_t)b * step.Hkv * kHeadDim);
      const i32x4* vs = reinterpret_cast<const i32x4*>(step.v_new + (size_t)b * step.Hkv * kHeadDim);
      for (int x = lane; x < nvec; x += 64) {
        reinterpret_cast<i32x4*>(step.k_cache + kv_row)[x] = ks[x];
        reinterpret_cast<i32x4*>(step.v_cache + kv_row)[x] = vs[x];
      }
      const int8_t* in = step.idx_new + (size_t)b * kIdxTokenBytes;
      int8_t* page_keys = step.idx_cache + (size_t)page * kIdxPageBytes;
      if (lane < 16)
        reinterpret_cast<i32x4*>(page_keys + row * kIdxTokenBytes)[lane] = reinterpret_cast<const i32x4*>(in)[lane];
      // new entry of slot row/4: the half holding that slot recomputes its 8 keys per lane
      const int slot = row / kTokensPerBlock;
      if (hf == (slot & 1)) {
        int sum[8];
        const int2 nw = *reinterpret_cast<const int2*>(in + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] = sbyte(e < 4 ? nw.x : nw.y, e & 3);
        for (int u = slot * kTokensPerBlock; u < row; ++u) {
          const int2 ow = *reinterpret_cast<const int2*>(page_keys + u * kIdxTokenBytes + 8 * c);
#pragma unroll
          for (int e = 0; e < 8; ++e) sum[e] += sbyte(e < 4 ? ow.x : ow.y, e & 3);
        }
        const i32x4 packed = {(sum[0] & 0xFFFF) | (sum[1] << 16), (sum[2] & 0xFFFF) | (sum[3] << 16),
                              (sum[4] & 0xFFFF) | (sum[5] << 16), (sum[6] & 0xFFFF) | (sum[7] << 16)};
        *reinterpret_cast<i32x4*>(reinterpret_cast<int8_t*>(pooled) + (size_t)page * kPooledPageBytes +
                                  slot * kPooledBlockBytes + 16 * c) = packed;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[k][i] = i == slot / 2 ? packed : v[k][i];
      }
    }
    int tot[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int a = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = v[k][i][e];   // a plain int first: a bit cast of the subscript itself read element 0
        a = __builtin_amdgcn_sdot2(__builtin_bit_cast(short2v, w), qd[e], a, false);
      }
      a = row16_sum(a);
      tot[i] = a + __shfl_xor(a, 16, 64);   // the half's other row
    }
    // lane c < 8 of each half writes block 2c + hf
    const int first = p * kSlotsPerPage;
    int mine = tot[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mine = c == i ? tot[i] : mine;
    const int blk = first + 2 * c + hf;
    if (c < 8 && blk < nblk) scores[(size_t)b * max_blocks + blk] = mine;
    if (page_max != nullptr) {
      int m = (int)0x80000000;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = first + 2 * i + hf < nblk ? max(m, tot[i]) : m;
      m = max(m, __shfl_xor(m, 32, 64));
      if (lane == 0) page_max[(size_t)b * max_pages + p] = m;
    }
  }
}

// Multi-token decode over the side cache: T (2..4) draft tokens per request, draft token t
// seeing the first L_b - (T-1-t) tokens. A wave scores one page for all T queries, with the
// lane layout of the scan above (lane 32*hf + c: keys 8c .. 8c+7 of block 2i + hf). A page
// that holds no position some draft token must not see is read once from the side cache; a
// page within T-1 tokens of L_b (at most two per request) is read from its int8 indexer rows
// instead, token by token, each token's dot product kept for the draft tokens that see it:
// the side-cache entries of its blocks pool the draft tokens' keys as well. Scores and page
// maxima of draft token t go to row b*T + t, as in the int8 multi-token scan.
template <int WAVES, int T>
__global__ __launch_bounds__(WAVES * 64) void index_score_pooled_multi_kernel(
    const int8_t* __restrict__ q_idx, const int16_t* __restrict__ pooled, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages, int max_blocks,
    int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  const int b = blockIdx.y, lane = lane_id(), wave = threadIdx.x >> 6;
  const int p = blockIdx.x * WAVES + wave;
  // length and page entry in one round trip, as in the single-token scans
  const int L = lens[b];
  const int page = page_table[(size_t)b * max_pages + __builtin_amdgcn_readfirstlane(min(p, max_pages - 1))];
  asm volatile("" ::"s"(page));
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (p >= npages) return;
  const int hf = lane >> 5, c = lane & 31;
  const int valid = L - p * kPageSize;                 // tokens of this page below L (>= 1)
  const bool mixed = valid < kPageSize + T - 1;        // the same for the whole wave
  int2 q8[T];                                          // query values 8c .. 8c+7, int8
#pragma unroll
  for (int t = 0; t < T; ++t) q8[t] = *reinterpret_cast<const int2*>(q_idx + ((size_t)b * T + t) * kIdxTokenBytes + 8 * c);
  int part[T][8];                                      // the lane's part of block 2i+hf's score
  if (!mixed) {
    i32x4 v[8];
    const int8_t* base = reinterpret_cast<const int8_t*>(pooled) + (size_t)page * kPooledPageBytes + 16 * lane;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + 1024 * i));
#pragma unroll
    for (int t = 0; t < T; ++t) {
      short2v qd[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = e < 2 ? q8[t].x : q8[t].y;
        const int k0 = 2 * (e & 1);
        qd[e] = short2v{(short)sbyte(w, k0), (short)sbyte(w, k0 + 1)};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int a = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int w = v[i][e];
          a = __builtin_amdgcn_sdot2(__builtin_bit_cast(short2v, w), qd[e], a, false);
        }
        part[t][i] = a;
      }
    }
  } else {
    const int8_t* rows = idx_cache + (size_t)page * kIdxPageBytes + 8 * c;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) part[t][i] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int u = 0; u < kTokensPerBlock; ++u) {
        const int row = kTokensPerBlock * (2 * i + hf) + u;   // row of the page
        const int2 kv = row < valid ? *reinterpret_cast<const int2*>(rows + row * kIdxTokenBytes) : int2{0, 0};
#pragma unroll
        for (int t = 0; t < T; ++t) {
          int d = __builtin_amdgcn_sdot4(kv.x, q8[t].x, 0, false);
          d = __builtin_amdgcn_sdot4(kv.y, q8[t].y, d, false);
          part[t][i] += row < valid - (T - 1 - t) ? d : 0;
        }
      }
  }
  // Sums over the 32 lanes of each half, T values per block. First the two 16-lane rows of a
  // half trade halves of the token range (row 0 keeps tokens [0, H), row 1 tokens [H, 2H); T
  // odd gets a zero token), so each row then sums H values per block instead of T.
  constexpr int H = (T + 1) / 2;
  const bool row1 = (lane >> 4) & 1;
  int red[H][8];
#pragma unroll
  for (int k = 0; k < H; ++k)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int lo = part[k][i], hi = H + k < T ? part[H + k][i] : 0;
      const int keep = row1 ? hi : lo, send = row1 ? lo : hi;
      red[k][i] = row16_sum(keep + __shfl_xor(send, 16, 64));
    }
  // red[k][i] in row r of half hf: draft token r*H + k, block 2i + hf. Lane cc = 8*k + j of
  // the row writes token r*H + k, block 2j + hf.
  const int first = p * kSlotsPerPage;
  const int cc = lane & 15, kq = cc >> 3, j = cc & 7, tq = (row1 ? H : 0) + kq;
  if (kq < H && tq < T) {
    int mine = red[0][0];
#pragma unroll
    for (int k = 0; k < H; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) mine = (kq == k && j == i) ? red[k][i] : mine;
    const int Lt = L - (T - 1 - tq);
    const int nblk = Lt > 0 ? (Lt + kTokensPerBlock - 1) / kTokensPerBlock : 0;
    const int blk = first + 2 * j + hf;
    if (blk < nblk) scores[((size_t)b * T + tq) * max_blocks + blk] = mine;
  }
  if (page_max != nullptr) {
#pragma unroll
    for (int k = 0; k < H; ++k) {
      const int t = (row1 ? H : 0) + k;
      const int Lt = L - (T - 1 - t);
      const int nblk = Lt > 0 ? (Lt + kTokensPerBlock - 1) / kTokensPerBlock : 0;
      int m = (int)0x80000000;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = first + 2 * i + hf < nblk ? max(m, red[k][i]) : m;
      m = max(m, __shfl_xor(m, 32, 64));          // the other half's blocks
      if (hf == 0 && cc == 0 && t < T) page_max[((size_t)b * T + t) * max_pages + p] = m;
    }
  }
}

constexpr int kSideWaves = 8;   // 8 pages per workgroup: the pooled scan ran 0.5-0.9 us faster than with 16

hipError_t launch_pool_build(const int8_t* idx_cache, const int32_t* page_table, const int32_t* lens, int B,
                             int max_pages, int16_t* pooled, hipStream_t stream) {
  const unsigned gx = (unsigned)((max_pages + kSideWaves - 1) / kSideWaves);
  hipLaunchKernelGGL(pool_build_kernel<kSideWaves>, dim3(gx, B), dim3(kSideWaves * 64), 0, stream, idx_cache,
                     page_table, lens, max_pages, pooled);
  return hipGetLastError();
}

hipError_t launch_cache_append(const void* k_new, const void* v_new, const int8_t* idx_new, const int32_t* write,
                               void* k_cache, void* v_cache, int8_t* idx_cache, int16_t* pooled,
                               const int32_t* page_table, const int32_t* lens, int B, int Hkv, int max_pages,
                               hipStream_t stream) {
  hipLaunchKernelGGL(cache_append_kernel, dim3(B), dim3(256), 0, stream, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), idx_new, write, static_cast<uint16_t*>(k_cache),
                     static_cast<uint16_t*>(v_cache), idx_cache, pooled, page_table, lens, Hkv, max_pages);
  return hipGetLastError();
}

template <int WAVES>
void launch_pooled_w(int B, hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const int8_t* q_idx,
                     const int16_t* pooled, const int32_t* page_table, const int32_t* lens, int max_pages,
                     int max_blocks, int32_t* scores, int32_t* page_max, const StepWrite& step) {
  const dim3 grid((unsigned)((max_pages + WAVES - 1) / WAVES), B);
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL((index_score_pooled_kernel<WAVES, 1>), grid, dim3(WAVES * 64), 0, stream, e0, e1, 0, q_idx,
                          const_cast<int16_t*>(pooled), page_table, lens, max_pages, max_blocks, scores, page_max,
                          step);
  else
    hipLaunchKernelGGL((index_score_pooled_kernel<WAVES, 1>), grid, dim3(WAVES * 64), 0, stream, q_idx,
                       const_cast<int16_t*>(pooled), page_table, lens, max_pages, max_blocks, scores, page_max, step);
}

// k_new == nullptr: the scan alone; otherwise it also makes the decode step's cache writes. One
// page per wave; a batch with few pages in all gets one-wave workgroups, so that its pages
// spread over many CUs.
template <int WAVES, int T>
void launch_pooled_multi_w(int B, hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const int8_t* q_idx,
                           const int16_t* pooled, const int8_t* idx_keys, const int32_t* page_table,
                           const int32_t* lens, int max_pages, int max_blocks, int32_t* scores, int32_t* page_max) {
  const dim3 grid((unsigned)((max_pages + WAVES - 1) / WAVES), B);
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL((index_score_pooled_multi_kernel<WAVES, T>), grid, dim3(WAVES * 64), 0, stream, e0, e1, 0,
                          q_idx, pooled, idx_keys, page_table, lens, max_pages, max_blocks, scores, page_max);
  else
    hipLaunchKernelGGL((index_score_pooled_multi_kernel<WAVES, T>), grid, dim3(WAVES * 64), 0, stream, q_idx, pooled,
                       idx_keys, page_table, lens, max_pages, max_blocks, scores, page_max);
}

template <int T>
void launch_pooled_multi(int B, hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const int8_t* q_idx,
                         const int16_t* pooled, const int8_t* idx_keys, const int32_t* page_table, const int32_t* lens,
                         int max_pages, int max_blocks, int32_t* scores, int32_t* page_max) {
  if ((long long)B * max_pages >= 256LL * kSideWaves)
    launch_pooled_multi_w<kSideWaves, T>(B, stream, e0, e1, q_idx, pooled, idx_keys, page_table, lens, max_pages,
                                         max_blocks, scores, page_max);
  else
    launch_pooled_multi_w<1, T>(B, stream, e0, e1, q_idx, pooled, idx_keys, page_table, lens, max_pages, max_blocks,
                                scores, page_max);
}

// T = 1: k_new == nullptr gives the scan alone; otherwise it also makes the decode step's cache
// writes (idx_cache is then where the new indexer row goes). T = 2..4: draft tokens, scored
// from the side cache and, on the pages holding draft positions, from idx_keys (the int8
// indexer cache); no writes.
hipError_t launch_index_score_pooled(const int8_t* q_idx, const int16_t* pooled, const int32_t* page_table,
                                     const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                                     int32_t* page_max, const void* k_new, const void* v_new, const int8_t* idx_new,
                                     const int32_t* write, void* k_cache, void* v_cache, int8_t* idx_cache, int Hkv,
                                     hipStream_t stream, int T, const int8_t* idx_keys) {
  const StepWrite step{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), idx_new, write,
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), idx_cache, Hkv};
  hipEvent_t e0, e1;   // kernel-timestamp events of qsa_time_next_scan, if set
  take_scan_events(&e0, &e1);
  if (T > 1) {
    switch (T) {
      case 2: launch_pooled_multi<2>(B, stream, e0, e1, q_idx, pooled, idx_keys, page_table, lens, max_pages,
                                     max_blocks, scores, page_max); break;
      case 3: launch_pooled_multi<3>(B, stream, e0, e1, q_idx, pooled, idx_keys, page_table, lens, max_pages,
                                     max_blocks, scores, page_max); break;
      case 4: launch_pooled_multi<4>(B, stream, e0, e1, q_idx, pooled, idx_keys, page_table, lens, max_pages,
                                     max_blocks, scores, page_max); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if ((long long)B * max_pages >= 256LL * kSideWaves)
    launch_pooled_w<kSideWaves>(B, stream, e0, e1, q_idx, pooled, page_table, lens, max_pages, max_blocks, scores,
                                page_max, step);
  else
    launch_pooled_w<1>(B, stream, e0, e1, q_idx, pooled, page_table, lens, max_pages, max_blocks, scores, page_max,
                       step);
  return hipGetLastError();
}

}  // namespace qsa
