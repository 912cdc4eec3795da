// topk_select.hip - K2: exact top-k micro-block selection per request.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: the best 512 blocks are kept. The order is strict (higher score, then lower
// block index), so exactly one set of K_b = min(k, n_b) blocks is correct; it is
// reported in ascending block order.
//
// One 1024-thread workgroup per request; nothing is shared between workgroups, so there
// is no atomic ticket, no device-scope fence and no workspace.
//   load    thread t holds the order-preserving keys u = uint32(score) ^ 0x80000000 of
//           blocks j = t + 1024*i (coalesced 4-byte loads; up to 64 per thread in
//           registers, more are re-read from memory on every pass).
//   range   [lo, hi] = [min u, max u] by block reduction.
//   narrow  repeat: histogram the keys inside [lo, hi] into 2048 LDS bins of width
//           2^shift (shift = bitlen(hi - lo) - 11, at least 0); the bin holding the
//           need-th largest key becomes the new [lo, hi]; need drops by the keys above
//           it. Stop when the bin's keys are all needed (then every key >= lo is kept) or
//           the bin is a single value T (then every key > T is kept plus the first `need`
//           keys equal to T in block order). Each pass shrinks the range 2^11-fold, so a
//           32-bit key needs at most 3 passes; adaptive bin widths keep LDS atomic
//           contention low for wide and for tie-heavy score distributions alike.
//   output  one ballot per (wave, slot) gives 64 consecutive blocks, so the kept/tie
//           masks land in LDS as 64-bit words without atomics; a block-wide prefix of
//           popcounts turns them into ascending ids.
// Requests with at most k blocks keep all of them.
#include "qsa_device.h"

namespace qsa {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRegSlots = 64;                    // keys held in registers per thread
constexpr int kSelBins = 2048;
constexpr int kMaxSelBlocks = 262144;            // contexts up to 1,048,576 tokens

__device__ __forceinline__ uint32_t score_key(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

struct SelShared {
  uint32_t hist[kSelBins + 64];   // + one dummy bin per lane for keys that are not counted
  int scan[kSelWaves + 1];
  uint32_t red[2][kSelWaves];
  int out[4];
};

// Block-wide min and max of x (every thread must call).
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SelShared& sh, uint32_t* gmn,
                                             uint32_t* gmx) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, d, 64));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, d, 64));
  }
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) { sh.red[0][wave] = mn; sh.red[1][wave] = mx; }
  __syncthreads();
  uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) { a = min(a, sh.red[0][w]); b = max(b, sh.red[1][w]); }
  *gmn = a;
  *gmx = b;
  __syncthreads();
}

// Bin holding the need-th largest key of the histogram: *beta and the number of keys in
// the bins above it. Every thread must call.
__device__ __forceinline__ void find_bucket(SelShared& sh, uint32_t need, int* beta, uint32_t* above) {
  constexpr int per = kSelBins / kSelThreads;  // 2 bins per thread
  const int t = threadIdx.x;
  const uint32_t c0 = sh.hist[t * per], c1 = sh.hist[t * per + 1];
  int total;
  const int excl = block_exclusive_scan<kSelThreads>((int)(c0 + c1), sh.scan, &total);
  uint32_t run = (uint32_t)(total - excl) - (c0 + c1);   // keys in bins above this thread's pair
  if (run < need && run + c1 >= need) { sh.out[0] = t * per + 1; sh.out[1] = (int)run; }
  run += c1;
  if (run < need && run + c0 >= need) { sh.out[0] = t * per; sh.out[1] = (int)run; }
  __syncthreads();
  *beta = sh.out[0];
  *above = (uint32_t)sh.out[1];
  __syncthreads();
}

template <bool kReg>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const int32_t* __restrict__ scores,
                                                                  const int32_t* __restrict__ lens,
                                                                  int max_blocks, int k,
                                                                  int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ sel_count) {
  extern __shared__ uint64_t s_bits[];  // [2][nw_max]: kept mask, tie mask
  __shared__ SelShared sh;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int n = (lens[b] + kTokensPerBlock - 1) / kTokensPerBlock;
  int32_t* out = sel + (size_t)b * k;

  if (n <= k) {  // every block is kept
    for (int i = t; i < k; i += kSelThreads) out[i] = i < n ? i : -1;
    if (t == 0) sel_count[b] = n;
    return;
  }
  const int K = k;
  const int32_t* s = scores + (size_t)b * max_blocks;
  const int nslots = (n + kSelThreads - 1) / kSelThreads;   // slots i with t + 1024*i < n
  const int nw = (n + 63) / 64;
  uint64_t* keep_bits = s_bits;
  uint64_t* tie_bits = s_bits + ((max_blocks + 63) / 64);

  // Every slot loop below is branch-free: a key that should not be counted goes to the
  // lane's own dummy bin, so no per-slot exec masks are kept and lanes never collide on
  // a dummy address.
  // Slots past the end (block t + 1024*i >= n) hold key 0. Such a key lies inside the
  // current range only when lo == 0, and then it lands in bin 0: the passes subtract the
  // known number of them there, and the kept mask is trimmed to n bits at the end. The
  // slot loops therefore carry no per-slot validity masks and no branches; a key that
  // is outside the range goes to the lane's own dummy bin (no address collisions).
  const uint32_t dummy = kSelBins + lane;
  const int nloop = kReg ? kRegSlots : nslots;
  const uint32_t n_pad = (uint32_t)(nloop * kSelThreads - n);
  uint32_t reg[kReg ? kRegSlots : 1];
  auto for_slots = [&](auto&& f) {
    if constexpr (kReg) {
#pragma unroll
      for (int i = 0; i < kRegSlots; ++i) f(i, reg[i]);
    } else {
      for (int i = 0; i < nslots; ++i) {
        const int j = t + kSelThreads * i;
        f(i, j < n ? score_key(s[j]) : 0u);
      }
    }
  };

  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  if constexpr (kReg) {
#pragma unroll
    for (int i = 0; i < kRegSlots; ++i) {
      const int j = t + kSelThreads * i;
      const uint32_t u = score_key(s[min(j, n - 1)]);
      reg[i] = j < n ? u : 0u;
      mn = min(mn, u);             // the clamped load repeats block n-1: harmless for min/max
      mx = max(mx, u);
    }
  } else {
    for (int i = 0; i < nslots; ++i) {
      const uint32_t u = score_key(s[min(t + kSelThreads * i, n - 1)]);
      mn = min(mn, u);
      mx = max(mx, u);
    }
  }
  uint32_t lo, hi;
  block_minmax(mn, mx, sh, &lo, &hi);

  uint32_t need = (uint32_t)K;
  bool all_of_bucket = false;
  while (lo != hi) {
    const int shift = max(0, 32 - __builtin_clz(hi - lo) - 11);
    for (int i = t; i < kSelBins; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t clo = lo, span_all = hi - lo;
    for_slots([&](int, uint32_t u) {
      const uint32_t d = u - clo;
      atomicAdd(&sh.hist[d <= span_all ? d >> shift : dummy], 1u);
    });
    __syncthreads();
    if (t == 0 && clo == 0) sh.hist[0] -= n_pad;
    __syncthreads();
    int beta;
    uint32_t above;
    find_bucket(sh, need, &beta, &above);
    const uint32_t count = sh.hist[beta];
    const uint32_t nlo = lo + ((uint32_t)beta << shift);
    const uint32_t span = (1u << shift) - 1u;
    hi = (hi - nlo < span) ? hi : nlo + span;
    lo = nlo;
    need -= above;
    __syncthreads();
    if (count == need) { all_of_bucket = true; break; }
  }

  // Kept and tie masks, one ballot per (wave, slot) covering blocks 1024*i + 64*wave ..
  // +63 (word 16*i + wave). Lane i%64 of the wave keeps the words of slot i (a select,
  // not a branch) and stores them once. Bits past block n-1 are cleared afterwards.
  {
    const uint32_t flo = lo, fhi = hi;
    const bool fall = all_of_bucket;
    uint64_t my_keep = 0, my_tie = 0;
    int my_slot = lane;
    auto store = [&](int slot) {
      const int w = kSelWaves * slot + wave;
      if (slot < nslots && w < nw) { keep_bits[w] = my_keep; tie_bits[w] = my_tie; }
    };
    for_slots([&](int i, uint32_t u) {
      const bool kept = fall ? (u >= flo) : (u > fhi);
      const bool tie = !fall & (u == flo);
      const uint64_t mk = __ballot(kept), mt = __ballot(tie);
      if constexpr (!kReg) {
        if ((i & 63) == 0 && i > 0) { store(my_slot); my_slot += 64; }
      }
      my_keep = (lane == (i & 63)) ? mk : my_keep;
      my_tie = (lane == (i & 63)) ? mt : my_tie;
    });
    store(my_slot);
  }
  __syncthreads();
  if (t == 0 && (n & 63)) {
    const uint64_t live = (1ull << (n & 63)) - 1ull;
    keep_bits[nw - 1] &= live;
    tie_bits[nw - 1] &= live;
  }
  __syncthreads();

  // Contiguous word ranges per thread keep block order through the prefix sums.
  const int wper = (nw + kSelThreads - 1) / kSelThreads;
  const int w0 = min(nw, t * wper), w1 = min(nw, w0 + wper);
  if (!all_of_bucket) {  // take the first `need` ties in block order
    int mine = 0;
    for (int w = w0; w < w1; ++w) mine += __builtin_popcountll(tie_bits[w]);
    int tot;
    int before = block_exclusive_scan<kSelThreads>(mine, sh.scan, &tot);
    for (int w = w0; w < w1; ++w) {
      uint64_t m = tie_bits[w], take = 0;
      while (m && before < (int)need) {
        take |= m & (~m + 1);
        m &= m - 1;
        ++before;
      }
      keep_bits[w] |= take;
    }
    __syncthreads();
  }
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __builtin_popcountll(keep_bits[w]);
  int tot;
  int pos = block_exclusive_scan<kSelThreads>(mine, sh.scan, &tot);
  for (int w = w0; w < w1; ++w) {
    uint64_t m = keep_bits[w];
    while (m) {
      const int j = w * 64 + __builtin_ctzll(m);
      m &= m - 1;
      if (pos < k) out[pos] = j;
      ++pos;
    }
  }
  for (int i = tot + t; i < k; i += kSelThreads) out[i] = -1;
  if (t == 0) sel_count[b] = min(tot, k);
}

size_t topk_workspace_bytes(int B, int max_blocks) {
  (void)B;
  (void)max_blocks;
  return 0;
}

hipError_t launch_topk_select(const int32_t* scores, const int32_t* lens, int B, int max_blocks, int k,
                              int32_t* sel, int32_t* sel_count, void* workspace, hipStream_t stream) {
  (void)workspace;
  const size_t lds = 2 * (size_t)((max_blocks + 63) / 64) * sizeof(uint64_t);
  if (max_blocks <= kRegSlots * kSelThreads)
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       max_blocks, k, sel, sel_count);
  else
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       max_blocks, k, sel, sel_count);
  return hipGetLastError();
}

}  // namespace qsa
