// index_score_mq.hip - K1 for many new tokens per request: int8 indexer scan on MFMA.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: keys are pooled into micro-blocks of 4 tokens and scored against the indexer
// query. With T new tokens per request (a prefill chunk), new token t is scored like a
// single decode query at length L_b - (T-1-t) (it sees itself and the tokens before it),
// into scores row b*T + t; the block score is the same integer as for one query.
#include "qsa_device.h"

namespace qsa {

// A prefill chunk (or any T up to 4096 new tokens) turns the scan into an int8 contraction,
// S[t][m] = sum_k key[t][k] * q[m][k] over the 256 key bytes, done on
// v_mfma_i32_16x16x64_i8: A = 16 key tokens x 64 bytes, B = 64 bytes x 16 queries, and lane
// (g4, i16) ends with the four accumulator values of MFMA rows 4*g4 .. 4*g4+3 for query i16.
// The tokens are dealt so that those rows are one micro-block: in token tile tt, MFMA row
// r = 4*g4 + v holds token 16*g4 + 4*tt + v, so the lane's rows are block 4*g4 + tt, the
// block score is the sum of its four values, and over the four tiles the lane holds the four
// consecutive blocks 4*g4 .. 4*g4+3 (one 16-byte store per lane; a query's 16 blocks of the
// page are 64 contiguous bytes). Grid (page groups, B), 8 waves per workgroup (two
// workgroups share a CU, so one's loads overlap the other's compute), one page per wave: the wave keeps its page's 64 keys in registers in the A layout (16 loads of 16 bytes;
// lane i16 of tile tt: token 16*(i16/4) + 4*tt + i16%4, bytes 64*s + 16*g4 .. +15) and runs
// every 16-query tile of the request against them, so the keys are read once. The queries go
// through LDS in chunks of kQueryChunk, loaded once per workgroup (the first chunk's loads
// are issued before the keys', and the page id comes by a scalar load, so neither waits on
// the other). Causal masking (query m sees tokens < L_b - T + 1 + m) is applied only on
// pages that reach into the new tokens.
constexpr int kMqWaves = 8;
constexpr int kQueryChunk = 64;    // queries staged in LDS at a time (17 KiB with padding)
constexpr int kQStride = kIdxTokenBytes / 16 + 1;   // 16-byte vectors per staged query

__global__ __launch_bounds__(kMqWaves * 64) void index_score_mq_kernel(
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages,
    int max_blocks, int T, int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  // Query m of the chunk at s_q[m * kQStride ..]: 16 vectors plus one of padding, so the 16
  // queries a wave reads at once start in different banks.
  __shared__ i32x4 s_q[kQueryChunk * kQStride];
  static_assert((kQueryChunk * kIdxTokenBytes / 16) % (kMqWaves * 64) == 0, "whole vectors per thread");
  const int b = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int p = blockIdx.x * kMqWaves + wave;
  // The page id is wave-uniform: a scalar load (its own counter, so the keys wait for it
  // and not for the query loads) at a clamped index, in bounds whatever the length, issued
  // together with the length's load (the empty asm keeps it ahead of the exit test).
  const int page = page_table[(size_t)b * max_pages + __builtin_amdgcn_readfirstlane(min(p, max_pages - 1))];
  const int L = lens[b];
  asm volatile("" ::"s"(page), "s"(L));
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (blockIdx.x * kMqWaves >= npages) return;   // the same for the whole workgroup
  const bool active = p < npages;                 // idle waves still join the barriers
  const int valid = L - p * kPageSize;
  // The first query chunk is loaded before the keys, so its latency overlaps theirs; it is
  // written to LDS once it arrives (the key loads stay in flight).
  constexpr int kQVecs = kQueryChunk * kIdxTokenBytes / 16;   // 16-byte vectors per chunk
  constexpr int kQPer = kQVecs / (kMqWaves * 64);
  const int8_t* qrow0 = q_idx + (size_t)b * T * kIdxTokenBytes;
  const int nq0 = min(kQueryChunk, T);
  i32x4 q0[kQPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int x = threadIdx.x + kMqWaves * 64 * j;
    const int lim = nq0 * kIdxTokenBytes / 16;      // loaded without a branch (clamped index)
    const i32x4 v = reinterpret_cast<const i32x4*>(qrow0)[min(x, lim - 1)];
    q0[j] = x < lim ? v : i32x4{0, 0, 0, 0};
  }
  i32x4 key[4][4];
  if (active) {
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
  for (int m0 = 0; m0 < T; m0 += kQueryChunk) {
    const int nq = min(kQueryChunk, T - m0);
    if (m0 == 0) {
#pragma unroll
      for (int j = 0; j < kQPer; ++j) {
        const int x = threadIdx.x + kMqWaves * 64 * j;
        s_q[(x >> 4) * kQStride + (x & 15)] = q0[j];
      }
    } else {
      __syncthreads();                             // the previous chunk is no longer read
      for (int x = threadIdx.x; x < kQVecs; x += kMqWaves * 64)
        s_q[(x >> 4) * kQStride + (x & 15)] =
            x < nq * kIdxTokenBytes / 16 ? reinterpret_cast<const i32x4*>(qrow0 + (size_t)m0 * kIdxTokenBytes)[x]
                                         : i32x4{0, 0, 0, 0};
    }
    __syncthreads();
    if (!active) continue;
    for (int qt = 0; qt < nq; qt += 16) {
      const int m = m0 + qt + i16;                 // this lane's query
      i32x4 qv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) qv[s] = s_q[(qt + i16) * kQStride + 4 * s + g4];
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

hipError_t launch_index_score_mq(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                                 const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                                 int32_t* page_max, int T, hipStream_t stream) {
  if (T < 1 || T > kMaxQueries) return hipErrorInvalidValue;
  const unsigned gm = (unsigned)((max_pages + kMqWaves - 1) / kMqWaves);
  hipLaunchKernelGGL(index_score_mq_kernel, dim3(gm, B), dim3(kMqWaves * 64), 0, stream, q_idx, idx_cache,
                     page_table, lens, max_pages, max_blocks, T, scores, page_max);
  return hipGetLastError();
}

}  // namespace qsa
