// index_score.hip - K1: int8 indexer scan, 4-token micro-block pooling, block scores.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: the indexer pools the keys of every 4 consecutive tokens and scores each pool.
// Block j of request b pools tokens 4j..4j+3 (those below L_b):
//     S[b][j] = sum_h sum_d q_idx[b][h][d] * sum_t key[t][h][d]
// The kernel forms the same integer by accumulating, token by token, int8 dot products
// against q_idx into the block's accumulator (sum_t dot(q, key_t) = dot(q, sum_t key_t)
// holds exactly in integer arithmetic), so the pooled key never has to be widened.
//
// Mapping. Grid (page groups, B): wave w of workgroup x scores page x*WAVES + w of
// request blockIdx.y (workgroups past the request's pages exit at once), one 16 KiB
// page = 16 blocks per wave; WAVES is 16, or 4 or 1 for batches with few pages in all:
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
// Multi-token decode (T draft tokens per request, T <= 4): the page is read once and scored
// against the T indexer queries q_idx[b][t]; draft token t sees the first L_b - (T-1-t)
// tokens, and its scores and page maxima go to row b*T + t.
#include <hip/hip_ext.h>

#include "qsa_device.h"

namespace qsa {

template <int WAVES, int T>
__global__ __launch_bounds__(WAVES * 64) void index_score_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages,
    int max_blocks, int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  const int b = blockIdx.y;
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int p = blockIdx.x * WAVES + wave;
  const int r4 = lane >> 4, c = lane & 15;
  // The length and this wave's page-table entry (a scalar load at a clamped index, in bounds
  // whatever the length) are loaded together, so the keys wait for one round trip, not for
  // the length and then the page. The empty asm takes the page as an input ahead of the
  // exit test; without it the compiler moves the page load (and the loads of the kernel
  // arguments it needs) past the test, a chain of dependent round trips.
  const int L = lens[b];
  const int page = page_table[(size_t)b * max_pages + __builtin_amdgcn_readfirstlane(min(p, max_pages - 1))];
  asm volatile("" ::"s"(page));
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (p >= npages) return;
  i32x4 qv[T];
#pragma unroll
  for (int t = 0; t < T; ++t)
    qv[t] = *reinterpret_cast<const i32x4*>(q_idx + ((size_t)b * T + t) * kIdxTokenBytes + 16 * c);
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

  // acc[t][r]: this lane's part of the score of block 4*r4 + r for draft token t, which sees
  // the first valid - (T-1-t) tokens of the page. Only a page within T-1 tokens of L holds
  // positions some draft token must not see; every other page takes the unmasked path.
  int acc[T][4];
  const bool masked = T > 1 && valid < kPageSize + T - 1;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int vt = valid - (T - 1 - t);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int a = 0;
      if (!masked) {   // one accumulation chain over the block's 4 tokens
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x4 v = x[4 * r + u];
          a = __builtin_amdgcn_sdot4(v.x, qv[t].x, a, false);
          a = __builtin_amdgcn_sdot4(v.y, qv[t].y, a, false);
          a = __builtin_amdgcn_sdot4(v.z, qv[t].z, a, false);
          a = __builtin_amdgcn_sdot4(v.w, qv[t].w, a, false);
        }
      } else {         // each token's dot product, kept when draft token t sees it
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const i32x4 v = x[4 * r + u];
          int d = __builtin_amdgcn_sdot4(v.x, qv[t].x, 0, false);
          d = __builtin_amdgcn_sdot4(v.y, qv[t].y, d, false);
          d = __builtin_amdgcn_sdot4(v.z, qv[t].z, d, false);
          d = __builtin_amdgcn_sdot4(v.w, qv[t].w, d, false);
          a += 16 * r4 + 4 * r + u < vt ? d : 0;
        }
      }
      acc[t][r] = row16_sum(a);
    }
  }

  // Lane c of each 16-lane row writes draft token c/4, block 4*r4 + c%4 (T*4 <= 16 lanes).
  const int tq = c >> 2, rq = c & 3;
  if (tq < T) {
    int v = acc[0][0];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) v = (tq == t && rq == r) ? acc[t][r] : v;
    const int Lt = L - (T - 1 - tq);
    const int nblk = (Lt + kTokensPerBlock - 1) / kTokensPerBlock;
    const int blk = p * kBlocksPerPage + 4 * r4 + rq;
    if (Lt > 0 && blk < nblk) scores[((size_t)b * T + tq) * max_blocks + blk] = v;
  }
  if (page_max) {
    const int first = p * kBlocksPerPage + 4 * r4;   // blocks of this DPP row
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int Lt = L - (T - 1 - t);
      const int nblk = Lt > 0 ? (Lt + kTokensPerBlock - 1) / kTokensPerBlock : 0;
      int m = (int)0x80000000;
#pragma unroll
      for (int r = 0; r < 4; ++r) m = first + r < nblk ? max(m, acc[t][r]) : m;
      m = max(m, __shfl_xor(m, 16, 64));
      m = max(m, __shfl_xor(m, 32, 64));
      if (lane == 0) page_max[((size_t)b * T + t) * max_pages + p] = m;
    }
  }
}

// Prefill-sized T (5 .. 4096 queries) is scored by the int8 MFMA kernel of index_score_mq.hip.
hipError_t launch_index_score_mq(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                                 const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                                 int32_t* page_max, int T, hipStream_t stream);

constexpr int kScoreWaves = 16;     // waves (pages) per workgroup when the batch has pages enough
constexpr long long kFillGroups = 256;   // workgroups that put every CU to work

namespace {
// Events that the next launch of index_score_kernel on this thread records at its own start
// and end (set by qsa_time_next_scan; used once, then cleared).
thread_local hipEvent_t g_scan_start = nullptr, g_scan_stop = nullptr;

template <int WAVES, int TT>
void launch_scan_w(int B, hipStream_t stream, const int8_t* q_idx, const int8_t* idx_cache,
                   const int32_t* page_table, const int32_t* lens, int max_pages, int max_blocks, int32_t* scores,
                   int32_t* page_max) {
  const dim3 grid((unsigned)((max_pages + WAVES - 1) / WAVES), B);
  const hipEvent_t e0 = g_scan_start, e1 = g_scan_stop;
  g_scan_start = g_scan_stop = nullptr;
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL((index_score_kernel<WAVES, TT>), grid, dim3(WAVES * 64), 0, stream, e0, e1, 0, q_idx,
                          idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max);
  else
    hipLaunchKernelGGL((index_score_kernel<WAVES, TT>), grid, dim3(WAVES * 64), 0, stream, q_idx, idx_cache,
                       page_table, lens, max_pages, max_blocks, scores, page_max);
}

// A small batch (few pages in all, e.g. one request of 4K tokens) gets smaller workgroups so
// that its pages spread over many CUs instead of being streamed by a handful of them.
template <int TT>
void launch_scan(int B, hipStream_t stream, const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                 const int32_t* lens, int max_pages, int max_blocks, int32_t* scores, int32_t* page_max) {
  const long long pages = (long long)B * max_pages;
  if (pages >= kFillGroups * kScoreWaves)
    launch_scan_w<kScoreWaves, TT>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores,
                                   page_max);
  else if (pages >= kFillGroups * 4)
    launch_scan_w<4, TT>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max);
  else
    launch_scan_w<1, TT>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max);
}
}  // namespace

void set_scan_events(hipEvent_t start, hipEvent_t stop) {
  g_scan_start = start;
  g_scan_stop = stop;
}

// The events set for the next scan launch of this thread (cleared): for the side-cache scan.
void take_scan_events(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_scan_start;
  *stop = g_scan_stop;
  g_scan_start = g_scan_stop = nullptr;
}

hipError_t launch_index_score(const int8_t* q_idx, const int8_t* idx_cache,
                              const int32_t* page_table, const int32_t* lens, int B,
                              int max_pages, int max_blocks, int32_t* scores, int32_t* page_max,
                              int T, hipStream_t stream) {
  switch (T) {
    case 1: launch_scan<1>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max); break;
    case 2: launch_scan<2>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max); break;
    case 3: launch_scan<3>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max); break;
    case 4: launch_scan<4>(B, stream, q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max); break;
    default:
      return launch_index_score_mq(q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks, scores,
                                   page_max, T, stream);
  }
  return hipGetLastError();
}

}  // namespace qsa
