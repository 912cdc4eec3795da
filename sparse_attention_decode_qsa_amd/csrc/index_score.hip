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
// Multi-token decode (T draft tokens per request, T <= 4): the page is read once and scored
// against the T indexer queries q_idx[b][t]; draft token t sees the first L_b - (T-1-t)
// tokens, and its scores and page maxima go to row b*T + t.
#include "qsa_device.h"

namespace qsa {

template <int WAVES, int T>
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

// ------------------------------------------------------------------ many queries (T > 4)
// A prefill chunk (or any T up to 4096 new tokens) turns the scan into an int8 contraction,
// S[t][m] = sum_k key[t][k] * q[m][k] over the 256 key bytes, done on
// v_mfma_i32_16x16x64_i8: A = 16 key tokens x 64 bytes, B = 64 bytes x 16 queries, and lane
// (g4, i16) ends with the four accumulator values of MFMA rows 4*g4 .. 4*g4+3 for query i16.
// The tokens are dealt so that those rows are one micro-block: in token tile tt, MFMA row
// r = 4*g4 + v holds token 16*g4 + 4*tt + v, so the lane's rows are block 4*g4 + tt, the
// block score is the sum of its four values, and over the four tiles the lane holds the four
// consecutive blocks 4*g4 .. 4*g4+3 (one 16-byte store per lane; a query's 16 blocks of the
// page are 64 contiguous bytes). Grid (page groups, B), 16 waves per workgroup, one page per
// wave: the wave keeps its page's 64 keys in registers in the A layout (16 loads of 16 bytes;
// lane i16 of tile tt: token 16*(i16/4) + 4*tt + i16%4, bytes 64*s + 16*g4 .. +15) and runs
// every 16-query tile of the request against them, so the keys are read once. The queries go
// through LDS in chunks of kQueryChunk, loaded once per workgroup. Causal masking (query m
// sees tokens < L_b - T + 1 + m) is applied only on pages that reach into the new tokens.
constexpr int kMqWaves = 16;
constexpr int kQueryChunk = 128;   // queries staged in LDS at a time (32 KiB)

__global__ __launch_bounds__(kMqWaves * 64) void index_score_mq_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages,
    int max_blocks, int T, int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  __shared__ i32x4 s_q[kQueryChunk * kIdxTokenBytes / 16];
  const int b = blockIdx.y;
  const int L = lens[b];
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (blockIdx.x * kMqWaves >= npages) return;   // the same for the whole workgroup
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int p = blockIdx.x * kMqWaves + wave;
  const bool active = p < npages;                 // idle waves still join the barriers
  const int valid = L - p * kPageSize;
  i32x4 key[4][4];
  if (active) {
    const int page = page_table[(size_t)b * max_pages + p];
    const int8_t* base = idx_cache + (size_t)page * kIdxPageBytes + 16 * g4;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tok = 16 * (i16 >> 2) + 4 * tt + (i16 & 3);
        key[tt][s] = tok < valid ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
                                       base + tok * kIdxTokenBytes + 64 * s))
                                 : i32x4{0, 0, 0, 0};
      }
  }
  const int L0 = L - T + 1;                        // query 0 sees tokens < L0
  const bool causal = active && p * kPageSize + kPageSize > L0;
  const int8_t* qrow0 = q_idx + (size_t)b * T * kIdxTokenBytes;
  for (int m0 = 0; m0 < T; m0 += kQueryChunk) {
    const int nq = min(kQueryChunk, T - m0);
    __syncthreads();                               // the previous chunk is no longer read
    for (int x = threadIdx.x; x < kQueryChunk * kIdxTokenBytes / 16; x += kMqWaves * 64)
      s_q[x] = x < nq * kIdxTokenBytes / 16 ? reinterpret_cast<const i32x4*>(qrow0 + (size_t)m0 * kIdxTokenBytes)[x]
                                            : i32x4{0, 0, 0, 0};
    __syncthreads();
    if (!active) continue;
    for (int qt = 0; qt < nq; qt += 16) {
      const int m = m0 + qt + i16;                 // this lane's query
      i32x4 qv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[s] = s_q[(qt + i16) * (kIdxTokenBytes / 16) + 4 * s + g4];
      const int Lm = L0 + m;
      const int nblk = m < T && Lm > 0 ? (Lm + kTokensPerBlock - 1) / kTokensPerBlock : 0;
      int pmax = (int)0x80000000;
      int sc[4];   // blocks 4*g4 + tt of the page for query m
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        i32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(key[tt][s], qv[s], acc, 0, 0, 0);
        const int pos = p * kPageSize + 16 * g4 + 4 * tt;   // first token of the block
        if (causal)
          sc[tt] = (pos < Lm ? acc[0] : 0) + (pos + 1 < Lm ? acc[1] : 0) + (pos + 2 < Lm ? acc[2] : 0) +
                   (pos + 3 < Lm ? acc[3] : 0);
        else
          sc[tt] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        if (p * kBlocksPerPage + 4 * g4 + tt < nblk) pmax = max(pmax, sc[tt]);
      }
      const int blk0 = p * kBlocksPerPage + 4 * g4;
      int32_t* row = scores + ((size_t)b * T + m) * max_blocks;
      if (blk0 + 3 < nblk) {
        *reinterpret_cast<i32x4*>(row + blk0) = i32x4{sc[0], sc[1], sc[2], sc[3]};
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (blk0 + tt < nblk) row[blk0 + tt] = sc[tt];
      }
      if (page_max) {
        pmax = max(pmax, __shfl_xor(pmax, 16, 64));
        pmax = max(pmax, __shfl_xor(pmax, 32, 64));
        if (g4 == 0 && m < T) page_max[((size_t)b * T + m) * max_pages + p] = pmax;
      }
    }
  }
}

constexpr int kScoreWaves = 16;

hipError_t launch_index_score(const int8_t* q_idx, const int8_t* idx_cache,
                              const int32_t* page_table, const int32_t* lens, int B,
                              int max_pages, int max_blocks, int32_t* scores, int32_t* page_max,
                              int T, hipStream_t stream) {
  const unsigned gx = (unsigned)((max_pages + kScoreWaves - 1) / kScoreWaves);
#define QSA_SCAN(TT)                                                                                      \
  hipLaunchKernelGGL((index_score_kernel<kScoreWaves, TT>), dim3(gx, B), dim3(kScoreWaves * 64), 0, stream, \
                     q_idx, idx_cache, page_table, lens, max_pages, max_blocks, scores, page_max)
  switch (T) {
    case 1: QSA_SCAN(1); break;
    case 2: QSA_SCAN(2); break;
    case 3: QSA_SCAN(3); break;
    case 4: QSA_SCAN(4); break;
    default: {
      if (T < 1 || T > kMaxQueries) return hipErrorInvalidValue;
      const unsigned gm = (unsigned)((max_pages + kMqWaves - 1) / kMqWaves);
      hipLaunchKernelGGL(index_score_mq_kernel, dim3(gm, B), dim3(kMqWaves * 64), 0, stream, q_idx, idx_cache,
                         page_table, lens, max_pages, max_blocks, T, scores, page_max);
    }
  }
#undef QSA_SCAN
  return hipGetLastError();
}

}  // namespace qsa
