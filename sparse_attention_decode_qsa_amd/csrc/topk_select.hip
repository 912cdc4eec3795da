// topk_select.hip - K2: exact top-k micro-block selection per request.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: the best 512 blocks are kept. The order is strict (higher score, then lower
// block index), so exactly one set of K_b = min(k, n_b) blocks is correct; it is
// reported in ascending block order.
//
// Method: radix selection on the order-preserving key u = uint32(score) ^ 0x80000000.
//   pass A  (topk_hist_kernel)  every workgroup histograms one chunk of 4096 scores
//           into 2048 bins of width 2^14 over u in [2^31 - 2^24, 2^31 + 2^24) (the range
//           of indexer scores; the two end bins also take anything beyond) and adds its
//           bins into the request's global histogram.
//   pass B  (topk_select_kernel) every workgroup finds, from the histogram, the bin
//           that holds the K_b-th key from the top ("bucket"), then writes two bitmaps
//           of its chunk: keys above the bucket (kept for sure) and keys inside it.
//           The last workgroup of the request to finish (an atomic ticket; nobody
//           waits) resolves the bucket exactly:
//             - it needs all its members, or it holds at most 256 of them: rank them
//               by (key desc, index asc) in LDS and keep the best;
//             - it spans one key value: the ties are taken in index order;
//             - otherwise histogram the members again over the bucket's own range,
//               narrowing it 2^11-fold, and repeat.
//           It then turns the "kept" bitmap into ascending block ids and clears the
//           histogram and ticket for the next call.
// Requests with at most k blocks keep all of them and touch no workspace.
#include "qsa_device.h"

namespace qsa {

constexpr int kTopkThreads = 256;
constexpr int kChunk = 4096;               // scores per workgroup
constexpr int kBins = 2048;
constexpr int kCap = 256;                  // bucket size resolved by ranking
constexpr uint32_t kLo0 = 0x80000000u - (1u << 24);
constexpr int kShift0 = 14;

struct TopkWs {
  uint32_t* hist;       // [B][kBins]
  uint32_t* ticket;     // [B]
  uint64_t* gt_bits;    // [B][nwords]
  uint64_t* in_bits;    // [B][nwords]
  int nwords;
};

__host__ __device__ inline size_t topk_nwords(int max_blocks) { return ((size_t)max_blocks + 63) / 64; }

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline size_t topk_ws_bytes(int B, int max_blocks) {
  const size_t nw = topk_nwords(max_blocks);
  return align256((size_t)B * kBins * 4) + align256((size_t)B * 4) + 2 * align256((size_t)B * nw * 8);
}

__host__ __device__ inline TopkWs topk_ws(void* base, int B, int max_blocks) {
  char* p = static_cast<char*>(base);
  const size_t nw = topk_nwords(max_blocks);
  TopkWs w;
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)B * kBins * 4);
  w.ticket = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)B * 4);
  w.gt_bits = reinterpret_cast<uint64_t*>(p);
  p += align256((size_t)B * nw * 8);
  w.in_bits = reinterpret_cast<uint64_t*>(p);
  w.nwords = (int)nw;
  return w;
}

__device__ __forceinline__ uint32_t score_key(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

__device__ __forceinline__ int bin0(uint32_t u) {
  if (u < kLo0) return 0;
  const uint32_t d = (u - kLo0) >> kShift0;
  return d > (uint32_t)(kBins - 1) ? kBins - 1 : (int)d;
}

// Key interval [lo, hi] of pass-A bin i.
__device__ __forceinline__ void bin0_range(int i, uint32_t* lo, uint32_t* hi) {
  *lo = i == 0 ? 0u : kLo0 + ((uint32_t)i << kShift0);
  *hi = i == kBins - 1 ? 0xFFFFFFFFu : kLo0 + ((uint32_t)(i + 1) << kShift0) - 1u;
}

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Within the histogram h[0..kBins) find the bin holding the need-th largest key:
// sets *beta, *above (count of keys in bins above beta). Every thread must call it.
__device__ void find_bucket(const uint32_t* h, uint32_t need, int* s_scan, int* beta,
                            uint32_t* above, int* s_out) {
  constexpr int per = kBins / kTopkThreads;  // 8 bins per thread
  const int t = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) local += (int)h[t * per + i];
  int total;
  const int excl = block_exclusive_scan<kTopkThreads>(local, s_scan, &total);
  uint32_t run = (uint32_t)(total - excl - local);  // keys in bins above this thread's range
#pragma unroll
  for (int i = per - 1; i >= 0; --i) {
    const uint32_t c = h[t * per + i];
    if (run < need && run + c >= need) { s_out[0] = t * per + i; s_out[1] = (int)run; }
    run += c;
  }
  __syncthreads();
  *beta = s_out[0];
  *above = (uint32_t)s_out[1];
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(
    const int32_t* __restrict__ scores, const int32_t* __restrict__ lens, int max_blocks, int k,
    uint32_t* __restrict__ hist) {
  const int b = blockIdx.y;
  const int n = (lens[b] + kTokensPerBlock - 1) / kTokensPerBlock;
  const int start = blockIdx.x * kChunk;
  if (n <= k || start >= n) return;
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kTopkThreads) h[i] = 0;
  __syncthreads();
  const int32_t* s = scores + (size_t)b * max_blocks + start;
  const int cnt = min(kChunk, n - start);
#pragma unroll 4
  for (int i = threadIdx.x; i < cnt; i += kTopkThreads) atomicAdd(&h[bin0(score_key(s[i]))], 1u);
  __syncthreads();
  uint32_t* gh = hist + (size_t)b * kBins;
  for (int i = threadIdx.x; i < kBins; i += kTopkThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
}

__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(
    const int32_t* __restrict__ scores, const int32_t* __restrict__ lens, int B, int max_blocks,
    int k, int32_t* __restrict__ sel, int32_t* __restrict__ sel_count, void* workspace) {
  const int b = blockIdx.y;
  const int n = (lens[b] + kTokensPerBlock - 1) / kTokensPerBlock;
  const int start = blockIdx.x * kChunk;
  int32_t* out = sel + (size_t)b * k;
  const int t = threadIdx.x;

  if (n <= k) {  // every block is kept
    if (start < n)
      for (int i = t; i < kChunk && start + i < n; i += kTopkThreads) out[start + i] = start + i;
    if (blockIdx.x == 0) {
      for (int i = n + t; i < k; i += kTopkThreads) out[i] = -1;
      if (t == 0) sel_count[b] = n;
    }
    return;
  }
  if (start >= n) return;

  TopkWs ws = topk_ws(workspace, B, max_blocks);
  const int32_t* s = scores + (size_t)b * max_blocks;
  uint32_t* gh = ws.hist + (size_t)b * kBins;
  uint64_t* gt = ws.gt_bits + (size_t)b * ws.nwords;
  uint64_t* in = ws.in_bits + (size_t)b * ws.nwords;
  const int K = k;

  __shared__ uint32_t h[kBins];
  __shared__ int s_scan[kTopkThreads / 64 + 1];
  __shared__ int s_out[4];
  __shared__ uint32_t s_ckey[kCap];
  __shared__ int s_cidx[kCap];
  __shared__ int s_flag;

  for (int i = t; i < kBins; i += kTopkThreads) h[i] = gh[i];
  __syncthreads();
  int beta;
  uint32_t above;
  find_bucket(h, (uint32_t)K, s_scan, &beta, &above, s_out);
  uint32_t lo, hi;
  bin0_range(beta, &lo, &hi);

  // Bitmaps of this chunk: one ballot per 64 consecutive blocks.
  {
    const int lane = lane_id(), wave = t >> 6;
    for (int grp = wave; grp < kChunk / 64; grp += kTopkThreads / 64) {
      const int j = start + grp * 64 + lane;
      bool g = false, m = false;
      if (j < n) {
        const uint32_t u = score_key(s[j]);
        g = u > hi;
        m = u >= lo && u <= hi;
      }
      const uint64_t mg = __ballot(g), mm = __ballot(m);
      const int w = (start >> 6) + grp;
      if (lane == 0 && start + grp * 64 < n) { gt[w] = mg; in[w] = mm; }
    }
  }

  // Ticket: the last workgroup of this request continues.
  const int nwg = (n + kChunk - 1) / kChunk;
  __threadfence();
  __syncthreads();
  if (t == 0) s_flag = atomicAdd(&ws.ticket[b], 1u) == (uint32_t)(nwg - 1);
  __syncthreads();
  if (!s_flag) return;
  __threadfence();

  const int nw = (n + 63) / 64;
  const int wper = (nw + kTopkThreads - 1) / kTopkThreads;  // contiguous words per thread
  const int w0 = min(nw, t * wper), w1 = min(nw, w0 + wper);
  uint32_t need = (uint32_t)K - above;  // still to take from the bucket
  uint32_t count = h[beta];

  for (;;) {
    if (count == need) {  // the whole bucket is kept
      for (int w = w0; w < w1; ++w) gt[w] = ld_agent(&gt[w]) | ld_agent(&in[w]);
      break;
    }
    if (count <= (uint32_t)kCap) {  // rank the members
      if (t == 0) s_out[2] = 0;
      __syncthreads();
      for (int w = w0; w < w1; ++w) {
        uint64_t m = ld_agent(&in[w]);
        while (m) {
          const int j = w * 64 + __builtin_ctzll(m);
          m &= m - 1;
          const int slot = atomicAdd(&s_out[2], 1);
          if (slot < kCap) { s_ckey[slot] = score_key(s[j]); s_cidx[slot] = j; }
        }
      }
      __syncthreads();
      const int c = min(s_out[2], kCap);
      if (t < c) {
        const uint32_t u = s_ckey[t];
        const int j = s_cidx[t];
        uint32_t rank = 0;
        for (int i = 0; i < c; ++i) {
          const uint32_t v = s_ckey[i];
          rank += (v > u) || (v == u && s_cidx[i] < j);
        }
        if (rank < need) atomicOr((unsigned long long*)&gt[j >> 6], 1ull << (j & 63));
      }
      break;
    }
    if (lo == hi) {  // one key value: ties in index order
      int mine = 0;
      for (int w = w0; w < w1; ++w) mine += __builtin_popcountll(ld_agent(&in[w]));
      int tot;
      int before = block_exclusive_scan<kTopkThreads>(mine, s_scan, &tot);
      for (int w = w0; w < w1; ++w) {
        uint64_t m = ld_agent(&in[w]), take = 0;
        while (m && before < (int)need) {
          const uint64_t bit = m & (~m + 1);
          take |= bit;
          m &= m - 1;
          ++before;
        }
        if (take) gt[w] = ld_agent(&gt[w]) | take;
      }
      break;
    }
    // Narrow the bucket: histogram its members over [lo, hi].
    const int shift = max(0, 32 - __builtin_clz(hi - lo) - 11);
    for (int i = t; i < kBins; i += kTopkThreads) h[i] = 0;
    __syncthreads();
    for (int w = w0; w < w1; ++w) {
      uint64_t m = ld_agent(&in[w]);
      while (m) {
        const int j = w * 64 + __builtin_ctzll(m);
        m &= m - 1;
        atomicAdd(&h[(score_key(s[j]) - lo) >> shift], 1u);
      }
    }
    __syncthreads();
    int beta2;
    uint32_t above2;
    find_bucket(h, need, s_scan, &beta2, &above2, s_out);
    const uint32_t nlo = lo + ((uint32_t)beta2 << shift);
    const uint32_t span = (shift >= 32) ? 0xFFFFFFFFu : ((1u << shift) - 1u);
    const uint32_t nhi = (hi - nlo < span) ? hi : nlo + span;
    for (int w = w0; w < w1; ++w) {
      uint64_t m = ld_agent(&in[w]), up = 0, keep = 0;
      uint64_t mm = m;
      while (mm) {
        const int bit = __builtin_ctzll(mm);
        mm &= mm - 1;
        const uint32_t u = score_key(s[w * 64 + bit]);
        if (u > nhi) up |= 1ull << bit;
        else if (u >= nlo) keep |= 1ull << bit;
      }
      if (up) gt[w] = ld_agent(&gt[w]) | up;
      in[w] = keep;
    }
    need -= above2;
    count = h[beta2];
    lo = nlo;
    hi = nhi;
    __threadfence_block();
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();

  // Kept bitmap -> ascending block ids.
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __builtin_popcountll(ld_agent(&gt[w]));
  int tot;
  int pos = block_exclusive_scan<kTopkThreads>(mine, s_scan, &tot);
  for (int w = w0; w < w1; ++w) {
    uint64_t m = ld_agent(&gt[w]);
    while (m) {
      const int j = w * 64 + __builtin_ctzll(m);
      m &= m - 1;
      if (pos < k) out[pos] = j;
      ++pos;
    }
  }
  for (int i = tot + t; i < k; i += kTopkThreads) out[i] = -1;
  if (t == 0) {
    sel_count[b] = min(tot, k);
    ws.ticket[b] = 0;
  }
  for (int i = t; i < kBins; i += kTopkThreads) gh[i] = 0;
}

size_t topk_workspace_bytes(int B, int max_blocks) { return topk_ws_bytes(B, max_blocks); }

hipError_t launch_topk_select(const int32_t* scores, const int32_t* lens, int B, int max_blocks,
                              int k, int32_t* sel, int32_t* sel_count, void* workspace,
                              hipStream_t stream) {
  const unsigned chunks = (unsigned)((max_blocks + kChunk - 1) / kChunk);
  TopkWs ws = topk_ws(workspace, B, max_blocks);
  hipLaunchKernelGGL(topk_hist_kernel, dim3(chunks, B), dim3(kTopkThreads), 0, stream, scores,
                     lens, max_blocks, k, ws.hist);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_select_kernel, dim3(chunks, B), dim3(kTopkThreads), 0, stream, scores,
                     lens, B, max_blocks, k, sel, sel_count, workspace);
  return hipGetLastError();
}

}  // namespace qsa
