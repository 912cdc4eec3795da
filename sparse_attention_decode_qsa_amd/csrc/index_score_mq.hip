// index_score_mq.hip - K1 for many new tokens per request: int8 indexer scan on MFMA.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: keys are pooled into micro-blocks of 4 tokens and scored against the indexer
// query. With T new tokens per request (a prefill chunk), new token t is scored like a
// single decode query at length L_b - (T-1-t) (it sees itself and the tokens before it),
// into scores row b*T + t; the block score is the same integer as for one query.
#include <hip/hip_ext.h>

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
// page are 64 contiguous bytes). Grid (page groups, B), one page per wave: the wave reads its
// page's 64 keys with 16 loads of 1 KiB each (four whole token rows per load), passes them
// once through its own LDS area into the A layout (lane i16 of tile tt, k-step s: token
// 16*(i16/4) + 4*tt + i16%4, bytes 64*s + 16*g4 .. +15), keeps them in registers and runs
// every 16-query tile of the request against them, so the keys are read once. Loading the A
// layout directly would make every load 16 pieces of 64 bytes, 256 bytes apart; on this GPU
// that made the scan 17-19% slower at up to 64 queries. The queries go through LDS in chunks
// of kQueryChunk, loaded once per workgroup (the first chunk's loads are issued before the
// keys', and the page id comes by a scalar load, so neither waits on the other). Causal
// masking (query m sees tokens < L_b - T + 1 + m) is applied only on pages that reach into
// the new tokens.
//
// Up to one chunk of queries (T <= kQueryChunk), 8-wave workgroups (two per CU) write each
// query's page maximum directly. With more, 16-wave workgroups fold the page maxima into LDS
// words and write a query's 16 consecutive page maxima together after each chunk (one 64-byte
// run instead of 16 separate 4-byte stores, which took nearly as long as the 755 MB of
// scores at T = 1024 on the 256K workload). On pages every query sees whole, a wave's four token tiles
// run as independent MFMA chains with no masking.
//
// From 5 to 64 queries the score rows go out as nontemporal stores: the selection reads them
// only on its candidate pages, and kept out of L2 and the MALL they leave that room to the
// attention's K/V rows (whole calls at the 256K workload: 8 queries 81.8 -> 80.9 us, 16
// queries 111.8 -> 108.0 us, 32 queries 162.2 -> 157.0 us, 64 queries 245.9 -> 240.5 us).
// With 2 to 4 draft queries they made the scan and the call slower (four queries 67.3 ->
// 69.0 us per call). Above 64 queries the effect changed sign from one GPU to the next (1,024
// correlated queries: -10 to +50 us per call of about 900 us; under a kernel trace the
// selection gained 19 us and the attention lost 7 us), so the 16-wave form stores plainly too.
hipError_t launch_index_score(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                              const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                              int32_t* page_max, int T, hipStream_t stream);   // index_score.hip
void take_scan_events(hipEvent_t* start, hipEvent_t* stop);                   // index_score.hip
constexpr long long kMqMinPages = 4096;   // batches from this many pages take the MFMA scan from T = 2
constexpr int kMaxDraftQueries = 4;   // up to here score rows are stored plainly (see store_scores)
constexpr int kQueryChunk = 64;    // queries staged in LDS at a time (17 KiB with padding)
constexpr int kQStride = kIdxTokenBytes / 16 + 1;   // 16-byte vectors per staged query

// One lane's 16-byte run of four block scores. NTS: a nontemporal store, so the score rows
// of a chunk (which the selection reads only on its candidate pages) do not take L2 and MALL
// space from the attention's K/V rows.
template <bool NTS>
__device__ __forceinline__ void store_scores(int32_t* dst, i32x4 v) {
  if constexpr (NTS) __builtin_nontemporal_store(v, reinterpret_cast<i32x4*>(dst));
  else *reinterpret_cast<i32x4*>(dst) = v;
}

// Scores of the page held in key (A layout, see above) for the nq queries of the chunk in
// s_q, 16 queries per step. FULL: every query sees all 64 tokens of the page, so no token or
// block is masked; the four token tiles' MFMA chains are independent and interleave. Page
// maxima: STAGE folds each query's into pm_slot (this wave's column of the chunk's LDS words,
// row stride WAVES); otherwise the lanes of a query combine theirs and one writes it to
// page_max.
template <int WAVES, bool STAGE, bool FULL, bool NTS>
__device__ __forceinline__ void score_query_tiles(const i32x4 (&key)[4][4], const i32x4* s_q, int m0, int nq,
                                                  int T, int L0, int p, int i16, int g4, int b, int max_blocks,
                                                  int max_pages, int32_t* __restrict__ scores, int* pm_slot,
                                                  int32_t* __restrict__ page_max) {
  const int blk0 = p * kBlocksPerPage + 4 * g4;   // this lane's first block of the page
  for (int qt = 0; qt < nq; qt += 16) {
    const int m = m0 + qt + i16;                   // this lane's query
    i32x4 qv[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[s] = s_q[(qt + i16) * kQStride + 4 * s + g4];
    i32x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(key[tt][s], qv[s], acc[tt], 0, 0, 0);
    int32_t* row = scores + ((size_t)b * T + m) * max_blocks;
    int sc[4];   // blocks 4*g4 + tt of the page for query m
    int pmax;
    if (FULL) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) sc[tt] = (acc[tt][0] + acc[tt][1]) + (acc[tt][2] + acc[tt][3]);
      pmax = max(max(sc[0], sc[1]), max(sc[2], sc[3]));
      if (m < T) store_scores<NTS>(row + blk0, i32x4{sc[0], sc[1], sc[2], sc[3]});
    } else {
      const int Lm = L0 + m;
      const int nblk = m < T && Lm > 0 ? (Lm + kTokensPerBlock - 1) / kTokensPerBlock : 0;
      pmax = (int)0x80000000;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int pos = p * kPageSize + 16 * g4 + 4 * tt;   // first token of the block
        sc[tt] = (pos < Lm ? acc[tt][0] : 0) + (pos + 1 < Lm ? acc[tt][1] : 0) + (pos + 2 < Lm ? acc[tt][2] : 0) +
                 (pos + 3 < Lm ? acc[tt][3] : 0);
        if (blk0 + tt < nblk) pmax = max(pmax, sc[tt]);
      }
      if (blk0 + 3 < nblk) {
        store_scores<NTS>(row + blk0, i32x4{sc[0], sc[1], sc[2], sc[3]});
      } else {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
          if (blk0 + tt < nblk) row[blk0 + tt] = sc[tt];
      }
    }
    if constexpr (STAGE) {
      if (pm_slot && m < T) atomicMax(pm_slot + (qt + i16) * WAVES, pmax);
    } else if (page_max) {
      pmax = max(pmax, __shfl_xor(pmax, 16, 64));
      pmax = max(pmax, __shfl_xor(pmax, 32, 64));
      if (g4 == 0 && m < T) page_max[((size_t)b * T + m) * max_pages + p] = pmax;
    }
  }
}

template <int WAVES, bool STAGE, bool NTS>
__global__ __launch_bounds__(WAVES * 64, 4) void index_score_mq_kernel(   // 4 waves per SIMD
    const int8_t* __restrict__ q_idx, const int8_t* __restrict__ idx_cache,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens, int max_pages,
    int max_blocks, int T, int32_t* __restrict__ scores, int32_t* __restrict__ page_max) {
  // Query m of the chunk at s_q[m * kQStride ..]: 16 vectors plus one of padding, so the 16
  // queries a wave reads at once start in different banks.
  __shared__ i32x4 s_q[kQueryChunk * kQStride];
  // STAGE: page maxima of a chunk, word q * WAVES + w = query q of the chunk, page w of the
  // workgroup; two buffers, so that one chunk's words are written out while the next fills.
  __shared__ int s_pm[STAGE ? 2 : 1][STAGE ? kQueryChunk * WAVES : 1];
  // Each wave's staging area for one token tile of its keys: 16 rows x 16 vectors, vector c of
  // row r at r * 16 + (c ^ r), so that the 16 rows a lane group writes or reads at once fall
  // in different banks.
  __shared__ i32x4 s_k[WAVES][16 * 16];
  static_assert((kQueryChunk * kIdxTokenBytes / 16) % (WAVES * 64) == 0, "whole vectors per thread");
  static_assert(kQueryChunk % 64 == 0, "whole page-maximum words per thread");
  const int b = blockIdx.y;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int p = __builtin_amdgcn_readfirstlane(blockIdx.x * WAVES + wave);   // wave-uniform
  // The page id is wave-uniform: a scalar load (its own counter, so the keys wait for it
  // and not for the query loads) at a clamped index, in bounds whatever the length, issued
  // together with the length's load (the empty asm keeps it ahead of the exit test).
  const int page = page_table[(size_t)b * max_pages + __builtin_amdgcn_readfirstlane(min(p, max_pages - 1))];
  const int L = lens[b];
  asm volatile("" ::"s"(page), "s"(L));
  const int npages = (L + kPageSize - 1) / kPageSize;
  if (blockIdx.x * WAVES >= npages) return;   // the same for the whole workgroup
  const bool active = p < npages;                 // idle waves still join the barriers
  const int valid = L - p * kPageSize;
  // The first query chunk is loaded before the keys, so its latency overlaps theirs; it is
  // written to LDS once it arrives (the key loads stay in flight).
  constexpr int kQVecs = kQueryChunk * kIdxTokenBytes / 16;   // 16-byte vectors per chunk
  constexpr int kQPer = kQVecs / (WAVES * 64);
  const int8_t* qrow0 = q_idx + (size_t)b * T * kIdxTokenBytes;
  const int nq0 = min(kQueryChunk, T);
  i32x4 q0[kQPer];
#pragma unroll
  for (int j = 0; j < kQPer; ++j) {
    const int x = threadIdx.x + WAVES * 64 * j;
    const int lim = nq0 * kIdxTokenBytes / 16;      // loaded without a branch (clamped index)
    const i32x4 v = reinterpret_cast<const i32x4*>(qrow0)[min(x, lim - 1)];
    q0[j] = x < lim ? v : i32x4{0, 0, 0, 0};
  }
  // The page's keys, read contiguously: load j brings tokens 4j .. 4j+3 (1 KiB; lane l holds
  // token 4j + l/16, bytes 16*(l%16) .. +15), and reaches the A layout through this wave's LDS
  // area.
  i32x4 key[4][4];
  i32x4 raw[16];
  if (active) {
    const int8_t* base = idx_cache + (size_t)page * kIdxPageBytes + 16 * lane;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      raw[j] = 4 * j + (lane >> 4) < valid
                   ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(base + j * 1024))
                   : i32x4{0, 0, 0, 0};
    // Token tile tt, MFMA row r = 4q + v: token 16q + 4tt + v, which load 4q + tt holds in lane
    // 16v + c (vector c). Written to the wave's area, read back in the A layout (lane (i16, g4)
    // of k-step s: row i16, vector 4s + g4). One wave's LDS operations run in order, so the
    // next tile's writes follow this tile's reads.
    i32x4* area = s_k[wave];
    const int rw = lane >> 4, cw = lane & 15;   // write side: row within the group, vector
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * q + rw;
        area[r * 16 + (cw ^ r)] = raw[4 * q + tt];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) key[tt][ks] = area[i16 * 16 + ((4 * ks + g4) ^ i16)];
    }
  }
  constexpr int kPmPer = kQueryChunk / 64;         // page-maximum words per thread and chunk
  if constexpr (STAGE) {
#pragma unroll
    for (int j = 0; j < kPmPer; ++j)
      s_pm[0][threadIdx.x + WAVES * 64 * j] = s_pm[1][threadIdx.x + WAVES * 64 * j] = (int)0x80000000;
  }
  // Writes out the page maxima of the chunk starting at query c0 (buffer buf) and clears them.
  auto flush_page_max = [&](int buf, int c0) {
    if constexpr (STAGE) {
#pragma unroll
      for (int j = 0; j < kPmPer; ++j) {
        const int w = threadIdx.x + WAVES * 64 * j;
        const int m = c0 + w / WAVES, pg = blockIdx.x * WAVES + w % WAVES;
        if (m < T && pg < npages) page_max[((size_t)b * T + m) * max_pages + pg] = s_pm[buf][w];
        s_pm[buf][w] = (int)0x80000000;
      }
    }
  };
  const int L0 = L - T + 1;                        // query 0 sees tokens < L0
  // A page every query sees whole (the usual case) takes a branch-free path; the page holding
  // the end of the context or reaching into the new tokens masks per token and per block.
  const bool full = active && (p + 1) * kPageSize <= L0;
  for (int m0 = 0; m0 < T; m0 += kQueryChunk) {
    const int nq = min(kQueryChunk, T - m0);
    if (m0 == 0) {
#pragma unroll
      for (int j = 0; j < kQPer; ++j) {
        const int x = threadIdx.x + WAVES * 64 * j;
        s_q[(x >> 4) * kQStride + (x & 15)] = q0[j];
      }
    } else {
      __syncthreads();                             // the previous chunk is no longer read
      if (page_max) flush_page_max(((m0 / kQueryChunk) - 1) & 1, m0 - kQueryChunk);   // a no-op unless STAGE
      for (int x = threadIdx.x; x < kQVecs; x += WAVES * 64)
        s_q[(x >> 4) * kQStride + (x & 15)] =
            x < nq * kIdxTokenBytes / 16 ? reinterpret_cast<const i32x4*>(qrow0 + (size_t)m0 * kIdxTokenBytes)[x]
                                         : i32x4{0, 0, 0, 0};
    }
    __syncthreads();
    if (!active) continue;
    int* pm_slot = nullptr;
    if constexpr (STAGE) {
      if (page_max) pm_slot = &s_pm[(m0 / kQueryChunk) & 1][wave];
    }
    if (full)
      score_query_tiles<WAVES, STAGE, true, NTS>(key, s_q, m0, nq, T, L0, p, i16, g4, b, max_blocks, max_pages, scores,
                                            pm_slot, page_max);
    else
      score_query_tiles<WAVES, STAGE, false, NTS>(key, s_q, m0, nq, T, L0, p, i16, g4, b, max_blocks, max_pages, scores,
                                             pm_slot, page_max);
  }
  if constexpr (STAGE) {
    if (page_max) {
      const int last = (T - 1) / kQueryChunk;      // the last chunk's maxima
      __syncthreads();
      flush_page_max(last & 1, last * kQueryChunk);
    }
  }
}

namespace {
template <int W, bool STAGE, bool NTS>
void launch_mq_w(hipStream_t stream, hipEvent_t e0, hipEvent_t e1, const int8_t* q_idx, const int8_t* idx_cache,
                 const int32_t* page_table, const int32_t* lens, int B, int max_pages, int max_blocks, int T,
                 int32_t* scores, int32_t* page_max) {
  const dim3 grid((unsigned)((max_pages + W - 1) / W), B);
  if (e0 != nullptr || e1 != nullptr)
    hipExtLaunchKernelGGL((index_score_mq_kernel<W, STAGE, NTS>), grid, dim3(W * 64), 0, stream, e0, e1, 0, q_idx,
                          idx_cache, page_table, lens, max_pages, max_blocks, T, scores, page_max);
  else
    hipLaunchKernelGGL((index_score_mq_kernel<W, STAGE, NTS>), grid, dim3(W * 64), 0, stream, q_idx, idx_cache,
                       page_table, lens, max_pages, max_blocks, T, scores, page_max);
}
}  // namespace

// start and stop, when not null, are recorded at the kernel's own start and end.
hipError_t launch_index_score_mq(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                                 const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                                 int32_t* page_max, int T, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
  if (T < 1 || T > kMaxQueries) return hipErrorInvalidValue;
  if (T <= kMaxDraftQueries)
    launch_mq_w<8, false, false>(stream, start, stop, q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks,
                                 T, scores, page_max);
  else if (T <= kQueryChunk)
    launch_mq_w<8, false, true>(stream, start, stop, q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks,
                                T, scores, page_max);
  else
    launch_mq_w<16, true, false>(stream, start, stop, q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks,
                                 T, scores, page_max);
  return hipGetLastError();
}

hipError_t launch_index_score_mq(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                                 const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                                 int32_t* page_max, int T, hipStream_t stream) {
  return launch_index_score_mq(q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks, scores, page_max, T,
                               stream, nullptr, nullptr);
}

// The scan of T queries per request. One query, and 2 to 4 queries on small batches, go to the
// int8 dot-product scan (index_score.hip), whose smaller workgroup forms spread a few pages
// over many CUs; from 2 queries on a batch of 4,096 pages or more goes to the MFMA scan, which
// reads the keys as whole 1 KiB pieces and takes its dot products off the vector ALUs (at the
// 256K workload, 2 / 3 / 4 queries: 34.9 / 36.4 / 38.7 us with dot products, 32.9 / 33.3 /
// 33.5 us on MFMA). A qsa_time_next_scan request is honoured by either.
hipError_t launch_multi_scan(const int8_t* q_idx, const int8_t* idx_cache, const int32_t* page_table,
                             const int32_t* lens, int B, int max_pages, int max_blocks, int32_t* scores,
                             int32_t* page_max, int T, hipStream_t stream) {
  if (T == 1 || (T <= 4 && (long long)B * max_pages < kMqMinPages))
    return launch_index_score(q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks, scores, page_max, T,
                              stream);
  hipEvent_t e0, e1;
  take_scan_events(&e0, &e1);
  return launch_index_score_mq(q_idx, idx_cache, page_table, lens, B, max_pages, max_blocks, scores, page_max, T,
                               stream, e0, e1);
}

}  // namespace qsa
