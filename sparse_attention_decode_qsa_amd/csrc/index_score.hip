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
// Mapping. The work is the flat list of pages of all requests (a prefix table over the
// page counts lives in LDS). One wave64 scores one 16 KiB page = 16 blocks per step:
//   lane = 16*r4 + c  (r4 = DPP row 0..3, c = 0..15)
//   load i (i = 0..15) of the lane reads the 16 bytes at offset 16*c of token
//   16*r4 + i of the page, so every load instruction reads four contiguous 256-byte
//   token rows. After 16 loads lane (r4, c) holds, for each of the blocks 4*r4 .. 4*r4+3,
//   the partial dot product of its 16 key bytes (head c/4, dims 16*(c%4)..+15) over the
//   block's 4 tokens. A 4-step DPP rotate-add inside each 16-lane row completes the sum
//   over the 256 key bytes of a token, and lanes c = 0..3 of row r4 store the scores of
//   blocks 4*r4 + c (64 contiguous bytes per page).
// Rows past L_b of the last page are read (the page is allocated) and masked to zero.
#include "qsa_device.h"

namespace qsa {

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void index_score_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int B,
    int max_pages, int max_blocks, int32_t* __restrict__ scores) {
  extern __shared__ int s_prefix[];  // [B + 1] exclusive prefix of page counts, + scan tmp
  int* s_tmp = s_prefix + B + 1;

  // Prefix table of page counts (contiguous ranges of requests per thread).
  {
    constexpr int NT = WAVES * 64;
    const int per = (B + NT - 1) / NT;
    const int lo = threadIdx.x * per, hi = min(B, lo + per);
    int local = 0;
    for (int i = lo; i < hi; ++i) local += (lens[i] + kPageSize - 1) / kPageSize;
    int total;
    int run = block_exclusive_scan<NT>(local, s_tmp, &total);
    for (int i = lo; i < hi; ++i) {
      s_prefix[i] = run;
      run += (lens[i] + kPageSize - 1) / kPageSize;
    }
    if (threadIdx.x == 0) s_prefix[B] = total;
    __syncthreads();
  }
  const int total_pages = s_prefix[B];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int r4 = lane >> 4, c = lane & 15;
  const int nworkers = gridDim.x * WAVES;

  int qb = -1;
  i32x4 qv = {0, 0, 0, 0};
  for (int g = blockIdx.x * WAVES + wave; g < total_pages; g += nworkers) {
    // request owning flat page g: the largest b with s_prefix[b] <= g
    int lo = 0, hi = B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= g) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int p = g - s_prefix[b];
    const int L = lens[b];
    const int page = page_table[(size_t)b * max_pages + p];
    if (b != qb) {
      qv = *reinterpret_cast<const i32x4*>(q_idx + (size_t)b * kIdxTokenBytes + 16 * c);
      qb = b;
    }
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
  }
}

constexpr int kScoreWaves = 4;

hipError_t launch_index_score(const int8_t* q_idx, const int8_t* idx_cache,
                              const int32_t* page_table, const int32_t* lens, int B,
                              int max_pages, int max_blocks, int32_t* scores, int num_cu,
                              hipStream_t stream) {
  const long long units = (long long)B * max_pages;            // upper bound on pages
  long long grid = (units + kScoreWaves - 1) / kScoreWaves;
  const long long cap = (long long)num_cu * 8;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  const size_t lds = (size_t)(B + 1 + kScoreWaves + 1) * sizeof(int);
  hipLaunchKernelGGL(index_score_kernel<kScoreWaves>, dim3((unsigned)grid), dim3(kScoreWaves * 64),
                     lds, stream, q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks,
                     scores);
  return hipGetLastError();
}

}  // namespace qsa
