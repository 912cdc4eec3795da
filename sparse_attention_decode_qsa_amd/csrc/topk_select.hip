// topk_select.hip - K2: exact top-k micro-block selection per request.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes", second
// paragraph: the best 512 blocks are kept. The order is strict (higher score, then lower
// block index), so exactly one set of K_b = min(k, n_b) blocks is correct; it is
// reported in ascending block order.
//
// One 1024-thread workgroup per request; nothing is shared between workgroups (no
// atomic ticket, no device-scope fence, no workspace). Keys are the order-preserving
// u = uint32(score) ^ 0x80000000. Thread t owns the R chunks c = t + 1024*r of 64
// consecutive blocks [64c, 64c + 64), so a per-thread 64-bit mask over a chunk is one
// word of a bitmap in block order.
// A short candidate list comes first, in one of two ways:
//   A. page maxima (written by the scan; used when there are at least k pages): the page
//      maxima are histogrammed over their [min, max] in 2048 bins and tau = the lower edge of
//      the bin holding the k-th largest. At least k pages reach tau, each with a block >= tau,
//      so the k-th key is >= tau and only pages reaching tau can hold kept blocks. Those pages
//      (about k; the bucket search counts them) are compacted by each wave for its own lanes
//      (ballots, no block barrier), their scores read by 4 lanes per page with every load of
//      a batch in flight, and the keys >= tau go to an LDS list (key, block) of at most 8192
//      entries (4096 past 256K tokens), each wave reserving its slots with one atomic after a
//      wave prefix sum.
//   B. otherwise, or if that list (or one wave's page list) would overflow:
//      1. load    the keys (in registers when R = 1, else re-read from memory) and the
//                 range [lo, hi] = [min u, max u] over the request.
//      2. sample  keys 0, 16, 32, 48 of every chunk are histogrammed over [lo, hi]; the
//                 lower edge of the bin holding their top 2*k*(samples/n) + 8 is a
//                 threshold tau that about 2k keys reach.
//      3. list    if between k and the list capacity keys reach tau, they go to the list;
//                 otherwise the narrowing below runs over every key.
// Then:
//   4. narrow  repeat: histogram the keys inside [lo, hi] into 2048 bins of width
//              2^shift (shift = bitlen(hi - lo) - 11, at least 0); the bin holding the
//              need-th largest key becomes [lo, hi]; need drops by the keys above it.
//              Stop when all keys of the bin are needed (keep every key >= lo) or the bin
//              is one value T (keep every key > T and the first `need` keys equal to T in
//              block order). At most 3 passes for 32-bit keys.
//   5. output  kept and tie masks per chunk; block prefix sums of their popcounts give
//              the tie ranks and the ascending output positions.
// The bucket search runs on one wave (DPP prefix sums) while the other waves clear the
// second histogram buffer; it and the block prefix sums cost one barrier each, reading
// their results from double-buffered LDS slots. Histogram loops over all keys are branch-free: a key that is
// not counted goes to the lane's own dummy bin. Requests with at most k blocks keep all of
// them. With T draft tokens per request (multi-token decode) workgroup r is the virtual
// request r = b*T + t, of length L_b - (T-1-t).
#include "qsa_device.h"

namespace qsa {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kChunk = 64;                       // blocks per chunk (one bitmap word)
constexpr int kSelBins = 2048;
// Candidate list capacity: 8192 when each thread owns one chunk (contexts up to 256K
// tokens), else 4096 (the mask words of longer contexts take the LDS).
constexpr int list_cap(int R) { return R == 1 ? 8192 : 4096; }
constexpr int kManyRequests = 512;               // from this many requests on, two workgroups per CU
constexpr int kWavePages = 256;                  // candidate pages one wave can hold
constexpr int kStridedOut = 8192;                // requests up to this many blocks write ids per block
constexpr int kMaxSelBlocks = 262144;            // contexts up to 1,048,576 tokens

__device__ __forceinline__ uint32_t score_key(int32_t s) { return (uint32_t)s ^ 0x80000000u; }

template <int R, int CAP>
struct SelShared {
  static constexpr int kListCap = CAP;
  uint32_t hbuf[2][kSelBins + 64];  // double-buffered histogram (+ one dummy bin per lane)
  uint32_t list_u[kListCap];
  int list_j[kListCap];
  int wpages[kSelWaves][kWavePages];     // per-wave candidate page ids of the page-maximum path
  alignas(16) int scan[2 * kSelWaves];   // block_exclusive_scan halves
  int wpre[kSelThreads];                 // output position of each mask word (short requests)
  uint32_t mm[2][2];                // (min, max) slots of the two block_minmax calls
  uint32_t sums[2];                 // slots of the two block_sum calls
  int fb[2][4];                     // find_bucket results, one slot per histogram buffer
  int list_n;
};


// Exclusive scan over the threads of a block of NT threads (NT a multiple of 256, <= 1024)
// with one barrier. `tmp` holds 2 * NT/64 ints of 16-byte aligned LDS and `buf` (0 or 1,
// the same in every thread, flipped by the call) picks the half this call uses: a call's
// wave totals are read after its barrier, and the half is written again only by the call
// after next, which comes after the next call's barrier. Returns the exclusive prefix and
// writes the block total to *total. Must be reached by every thread of the block.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int& buf, int* total) {
  constexpr int NW = NT / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x);
  int* h = tmp + buf * NW;
  if (lane == 63) h[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w4 = 0; w4 < NW / 4; ++w4) {
    const i32x4 v = reinterpret_cast<const i32x4*>(h)[w4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int w = 4 * w4 + e;
      before += w < wave ? v[e] : 0;
      all += v[e];
    }
  }
  buf ^= 1;
  *total = all;
  return before + inc - x;
}

// f(e) for the register slots e = 0 .. nvmax-1, unrolled in groups of 8 (so every index
// is a constant and the register array stays in registers) with a wave-uniform exit after
// the last group that holds a valid slot: a short request runs one or two groups, not 64.
template <typename F>
__device__ __forceinline__ void for_slots(int nvmax, F&& f) {
#pragma unroll
  for (int g = 0; g < kChunk / 8; ++g) {
    if (8 * g >= nvmax) break;
#pragma unroll
    for (int i = 0; i < 8; ++i) f(8 * g + i);
  }
}

// Block-wide min and max into slot sh.mm[slot], which thread 0 set to (~0, 0) before an
// earlier barrier (every thread must call; one barrier; the slot is not reused).
template <typename SH>
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx, SH& sh, int slot, uint32_t* gmn,
                                             uint32_t* gmx) {
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane_id() == 0) { atomicMin(&sh.mm[slot][0], mn); atomicMax(&sh.mm[slot][1], mx); }
  __syncthreads();
  *gmn = sh.mm[slot][0];
  *gmx = sh.mm[slot][1];
}

// Block-wide sum into slot sh.sums[slot], which thread 0 set to 0 before an earlier barrier
// (every thread must call; one barrier; the slot is not reused).
template <typename SH>
__device__ __forceinline__ uint32_t block_sum(uint32_t x, SH& sh, int slot) {
  x = wave_sum(x);
  if (lane_id() == 0 && x) atomicAdd(&sh.sums[slot], x);
  __syncthreads();
  return sh.sums[slot];
}

// Bin of the complete histogram holding the need-th largest key, the number of keys in
// the bins above it and in the bin itself (*beta = -1 when it holds fewer than `need`).
// Wave 0 searches (each lane sums 32 bins, a reverse wave scan finds the lane, that lane
// walks its bins) while the other threads clear the other histogram buffer; then the
// buffers swap. The result goes through slot sh.fb[hsel]: the next call writes the other
// slot, and the call after it comes after that call's barrier, when every thread has read
// this one. Every thread must call it; it costs one barrier.
template <typename SH>
__device__ __forceinline__ void find_bucket(SH& sh, int& hsel, uint32_t need, int* beta,
                                            uint32_t* above, uint32_t* count = nullptr) {
  constexpr int per = kSelBins / 64;
  const int t = threadIdx.x, lane = lane_id();
  const uint32_t* h = sh.hbuf[hsel];
  uint32_t* other = sh.hbuf[hsel ^ 1];
  if (t < 64) {
    // Lane l sums the 32 bins of group g = 63 - l, starting at a rotated offset so the 64
    // lanes read from distinct banks; a prefix sum over the lanes is then the number of
    // keys in group g and every group above it.
    const int g = 63 - lane;
    uint32_t c = 0;
#pragma unroll 8
    for (int i = 0; i < per; ++i) c += h[g * per + ((i + g) & (per - 1))];
    const uint32_t suf = (uint32_t)wave_inclusive_scan((int)c);
    const uint64_t hit = __ballot(suf - c < need && suf >= need);
    if (hit == 0) {
      if (lane == 0) { sh.fb[hsel][0] = -1; sh.fb[hsel][1] = 0; sh.fb[hsel][2] = 0; }
    } else {
      const int L = __builtin_ctzll(hit);
      const int G = 63 - L;
      const uint32_t runG = (uint32_t)__builtin_amdgcn_readlane((int)(suf - c), L);   // keys above group G
      // The wave walks group G's 32 bins from the top: lane l < 32 holds bin 32G + 31 - l.
      const uint32_t v = lane < per ? h[G * per + (per - 1 - lane)] : 0u;
      const uint32_t sv = (uint32_t)wave_inclusive_scan((int)v);
      const bool mine = lane < per && runG + sv - v < need && runG + sv >= need;
      if (mine) { sh.fb[hsel][0] = G * per + (per - 1 - lane); sh.fb[hsel][1] = (int)(runG + sv - v); sh.fb[hsel][2] = (int)v; }
    }
  } else {
    for (int i = t - 64; i < kSelBins + 64; i += kSelThreads - 64) other[i] = 0;
  }
  __syncthreads();
  *beta = sh.fb[hsel][0];
  *above = (uint32_t)sh.fb[hsel][1];
  if (count) *count = (uint32_t)sh.fb[hsel][2];
  hsel ^= 1;   // every thread flips its own copy: the cleared buffer is filled next
}

__device__ __forceinline__ int shift_for(uint32_t lo, uint32_t hi) {
  return max(0, 32 - __builtin_clz(hi - lo) - 11);
}

// One narrowing step on a complete histogram of the keys in [lo, hi]. Returns true when
// the bucket's keys are exactly the ones still needed.
template <typename SH>
__device__ __forceinline__ bool narrow_step(SH& sh, int& hsel, int shift, uint32_t* lo, uint32_t* hi,
                                            uint32_t* need) {
  int beta;
  uint32_t above;
  uint32_t count;
  find_bucket(sh, hsel, *need, &beta, &above, &count);
  const uint32_t nlo = *lo + ((uint32_t)beta << shift);
  const uint32_t span = (1u << shift) - 1u;
  *hi = (*hi - nlo < span) ? *hi : nlo + span;
  *lo = nlo;
  *need -= above;
  return count == *need;
}

// Narrow [lo, hi] over the LDS candidate list (all candidates are >= lo), then write the
// kept and tie masks of the candidates into the per-chunk words (zero on entry).
template <int R, int CAP>
__device__ __forceinline__ void narrow_list_and_mark(SelShared<R, CAP>& sh, int& hsel, uint32_t ncand, uint32_t lo, uint32_t hi,
                                                     uint32_t* need_io, bool* all_io, uint32_t* lo_out,
                                                     uint64_t* kept_w, uint64_t* tie_w) {
  const int t = threadIdx.x;
  uint32_t need = *need_io;
  bool all_of_bucket = false;
  while (lo != hi) {
    const int shift = shift_for(lo, hi);
    for (int i = t; i < (int)ncand; i += kSelThreads) {
      const uint32_t u = sh.list_u[i];
      if (u >= lo && u <= hi) atomicAdd(&sh.hbuf[hsel][(u - lo) >> shift], 1u);
    }
    __syncthreads();
    if (narrow_step(sh, hsel, shift, &lo, &hi, &need)) { all_of_bucket = true; break; }
  }
  // kept_w and tie_w were cleared at kernel start
  for (int i = t; i < (int)ncand; i += kSelThreads) {
    const uint32_t u = sh.list_u[i];
    const int j = sh.list_j[i];
    const uint64_t bit = 1ull << (j & 63);
    if (all_of_bucket ? u >= lo : u > hi) atomicOr((unsigned long long*)&kept_w[j >> 6], bit);
    else if (!all_of_bucket && u == lo) atomicOr((unsigned long long*)&tie_w[j >> 6], bit);
  }
  *need_io = need;
  *all_io = all_of_bucket;
  *lo_out = lo;
}

template <int R, int CAP = list_cap(R)>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(const int32_t* __restrict__ scores,
                                                                  const int32_t* __restrict__ lens,
                                                                  const int32_t* __restrict__ page_max,
                                                                  int max_blocks, int max_pages, int k,
                                                                  int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ sel_count, int T) {
  extern __shared__ uint64_t s_words[];  // [2][1024*R]: kept and tie masks per chunk
  __shared__ SelShared<R, CAP> sh;
  constexpr int kListCap = CAP;
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = lane_id();
  // The page maxima are loaded at clamped indices (in bounds whatever the length) together
  // with the length, so they do not wait for it; entries past the request's pages are masked
  // where they are used. The loads take no branch (without page maxima they read lens[0],
  // unused), and the empty asm statements keep them ahead of the early exit.
  constexpr int PV = 4 * R;                      // page maxima per thread (np <= 4096*R)
  const int32_t* pm = page_max != nullptr ? page_max + (size_t)b * max_pages : lens;
  const int pm_last = page_max != nullptr ? max_pages - 1 : 0;
  const int len = draft_length(lens, b, T);
  int32_t pm_raw[PV];
#pragma unroll
  for (int i = 0; i < PV; ++i) pm_raw[i] = pm[min(t + kSelThreads * i, pm_last)];
  asm volatile("" ::"s"(len));
#pragma unroll
  for (int i = 0; i < PV; ++i) asm volatile("" ::"v"(pm_raw[i]));
  uint32_t pv[PV];
#pragma unroll
  for (int i = 0; i < PV; ++i) pv[i] = score_key(pm_raw[i]);
  const int n = (len + kTokensPerBlock - 1) / kTokensPerBlock;
  int32_t* out = sel + (size_t)b * k;

  if (n <= k) {  // every block is kept
    for (int i = t; i < k; i += kSelThreads) out[i] = i < n ? i : -1;
    if (t == 0) sel_count[b] = n;
    return;
  }
  const int32_t* s = scores + (size_t)b * max_blocks;
  uint64_t* kept_w = s_words;
  uint64_t* tie_w = s_words + kSelThreads * R;
  const uint32_t dummy = kSelBins + lane;
  constexpr int kU = R == 1 ? kChunk : 1;   // full unroll only when the keys sit in registers

  uint32_t need = (uint32_t)k;
  bool all_of_bucket = false;
  bool masks_done = false;
  uint32_t lo = 0, hi = 0;
  int hsel = 0;   // histogram buffer being filled; the other one is cleared by find_bucket

  // A. Page maxima (when given and there are at least k pages): one histogram of the page
  // maxima over [min, max]; tau = the lower edge of the bin holding the k-th largest. At
  // least k pages reach tau, each with a block >= tau, so the k-th key is >= tau, and only
  // the blocks of pages reaching tau can be kept. Their loads are issued before the
  // histogram is cleared, so the two overlap.
  const int np = (n + kBlocksPerPage - 1) / kBlocksPerPage;
  const bool use_pm = page_max != nullptr && np >= k;
  if (use_pm) {
#pragma unroll
    for (int i = 0; i < PV; ++i) pv[i] = t + kSelThreads * i < np ? pv[i] : 0u;
  }
  for (int i = t; i < kSelBins + 64; i += kSelThreads) sh.hbuf[0][i] = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) { kept_w[t + kSelThreads * r] = 0; tie_w[t + kSelThreads * r] = 0; }
  if (t == 0) {
    sh.mm[0][0] = sh.mm[1][0] = 0xFFFFFFFFu;
    sh.mm[0][1] = sh.mm[1][1] = 0u;
    sh.sums[0] = sh.sums[1] = 0u;
    sh.list_n = 0;
  }
  __syncthreads();

  bool have_list = false;
  uint32_t ncand = 0;
  if (use_pm) {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int i = 0; i < PV; ++i) {
      const int pidx = t + kSelThreads * i;
      mn = min(mn, pidx < np ? pv[i] : 0xFFFFFFFFu);
      mx = max(mx, pv[i]);
    }
    uint32_t plo, phi;
    block_minmax(mn, mx, sh, 0, &plo, &phi);
    hi = phi;                                    // the largest page maximum is the largest key
    uint32_t tau = plo;
    int ncp = np;                                // pages whose maximum reaches tau
    if (plo != phi) {
      const int shift = shift_for(plo, phi);
#pragma unroll
      for (int i = 0; i < PV; ++i)
        atomicAdd(&sh.hbuf[hsel][t + kSelThreads * i < np ? (pv[i] - plo) >> shift : dummy], 1u);
      __syncthreads();
      int beta;
      uint32_t above, count;
      find_bucket(sh, hsel, (uint32_t)k, &beta, &above, &count);
      tau = plo + ((uint32_t)beta << shift);
      ncp = (int)(above + count);
    }
    // B. candidate blocks. Each wave compacts the pages of its lanes that reach tau into its
    // own LDS list (ballots, no block barrier; more than kWavePages in one wave counts as an
    // overflow), then reads them 4 lanes per page with one 16-byte load each, 16 pages per
    // step and every step's load in flight before any key is used, and appends the keys
    // >= tau to the block's LDS list with one reservation per wave and step. Order in the
    // list does not matter. Each such page adds at least one key, so more than kListCap
    // pages go straight to the fallback.
    if (ncp <= kListCap) {
      const int wave = t >> 6, sub = lane >> 2, q4 = lane & 3;
      int* wp = sh.wpages[wave];
      int nwp = 0;                               // wave-uniform
#pragma unroll
      for (int i = 0; i < PV; ++i) {
        const bool f = (t + kSelThreads * i < np) & (pv[i] >= tau);
        const uint64_t m = __ballot(f);
        const int pos = nwp + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (f && pos < kWavePages) wp[pos] = t + kSelThreads * i;
        nwp += __builtin_popcountll(m);
      }
      if (nwp > kWavePages) {
        if (lane == 0) atomicAdd(&sh.list_n, kListCap + 1);   // overflow: the list is not used
        nwp = 0;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      constexpr int kBatch = 4;
      for (int st0 = 0; st0 < nwp; st0 += 16 * kBatch) {
        int j0[kBatch];
        i32x4 v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const int ci = st0 + 16 * q + sub;
          j0[q] = -1;
          v[q] = i32x4{0, 0, 0, 0};
          if (ci < nwp) {
            const int j = kBlocksPerPage * wp[ci] + 4 * q4;
            if (j < n) { j0[q] = j; v[q] = *reinterpret_cast<const i32x4*>(s + j); }
          }
        }
        // Lane candidates (0..16 per batch) -> one wave prefix sum, then one list
        // reservation per wave for the whole batch; each lane writes its run of slots.
        uint32_t cm[kBatch];
        int c = 0;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          uint32_t m4 = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m4 |= (uint32_t)(j0[q] >= 0 && j0[q] + e < n && score_key(v[q][e]) >= tau) << e;
          cm[q] = m4;
          c += __builtin_popcount(m4);
        }
        const int incl = wave_inclusive_scan(c);
        int base = 0;
        if (lane == 63 && incl) base = atomicAdd(&sh.list_n, incl);
        int slot = __builtin_amdgcn_readlane(base, 63) + incl - c;
#pragma unroll
        for (int q = 0; q < kBatch; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if ((cm[q] >> e) & 1u) {
              if (slot < kListCap) { sh.list_u[slot] = score_key(v[q][e]); sh.list_j[slot] = j0[q] + e; }
              ++slot;
            }
      }
    }
    __syncthreads();
    ncand = (uint32_t)sh.list_n;   // list_n is written again only after later barriers
    if (ncp <= kListCap && ncand <= (uint32_t)kListCap) {
      have_list = true;
      lo = tau;
    }
  }

  // Sample path and full fallback over every key. With R = 1 the keys sit in registers,
  // strided: thread t holds blocks t + 1024*e (e = 0..63), so the loads are coalesced, every
  // thread has a share of a short request, and block t + 1024*e falls in mask word
  // wave + 16*e at bit lane (one ballot per slot gives a whole word). With R > 1 thread t
  // owns the chunks c = t + 1024*r of 64 consecutive blocks and reads its keys again.
  uint32_t reg[R == 1 ? kChunk : 1];
  int nv[R];   // valid slots e: R = 1: t + 1024*e < n; R > 1: 64*c + e < n
#pragma unroll
  for (int r = 0; r < R; ++r)
    nv[r] = R == 1 ? (n > t ? min(kChunk, (n - t + kSelThreads - 1) / kSelThreads) : 0)
                   : min(kChunk, max(0, n - kChunk * (t + kSelThreads * r)));
  auto key = [&](int r, int e) -> uint32_t {
    if constexpr (R == 1) {
      (void)r;
      return reg[e];
    } else {
      return score_key(s[min(kChunk * (t + kSelThreads * r) + e, n - 1)]);
    }
  };
  auto blk = [&](int r, int e) -> int {
    return R == 1 ? t + kSelThreads * e : kChunk * (t + kSelThreads * r) + e;
  };
  if (!have_list) {
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    // R = 1: the wave's largest slot count (lane 0 has it); every loop over the register
    // slots stops there, so slots past it are never read.
    const int nvmax = R == 1 ? __builtin_amdgcn_readfirstlane(nv[0]) : 0;
    if constexpr (R == 1) {
      // up to 64 coalesced loads of 4 bytes (a wave reads 256 contiguous bytes per slot);
      // slots at or past n are not loaded.
      for_slots(nvmax, [&](int e) {
        const int j = t + kSelThreads * e;
        reg[e] = j < n ? score_key(s[j]) : 0u;
      });
      for_slots(nvmax, [&](int e) {
        const bool ok = e < nv[0];
        mn = min(mn, ok ? reg[e] : 0xFFFFFFFFu);
        mx = max(mx, ok ? reg[e] : 0u);
      });
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
        for (int e = 0; e < nv[r]; ++e) { const uint32_t u = key(r, e); mn = min(mn, u); mx = max(mx, u); }
    }
    block_minmax(mn, mx, sh, 1, &lo, &hi);

    if (lo != hi) {
      // sample one key in 16: with R = 1 the slots e with e % 16 == (t / 16) % 16 (four per
      // thread, spread over the context), with R > 1 keys 0, 16, 32, 48 of every chunk.
      int shift = shift_for(lo, hi);
      uint32_t mine = 0;
      // With n <= 2k + 128 the sample's threshold would keep every key (its target count,
      // 2k*nsamp/n + 8, reaches nsamp), so the sample is skipped and tau = lo.
      const bool sample = n > 2 * k + 128;
      if (!sample) {
        // nothing: every key is a candidate
      } else if constexpr (R == 1) {
        const int c16 = (t >> 4) & 15;
        for_slots(nvmax, [&](int e) {
          if ((e & 15) == c16) {
            const bool ok = e < nv[0];
            mine += ok;
            atomicAdd(&sh.hbuf[hsel][ok ? (reg[e] - lo) >> shift : dummy], 1u);
          }
        });
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < kChunk; e += 16) {
            const bool ok = e < nv[r];
            mine += ok;
            atomicAdd(&sh.hbuf[hsel][ok ? (key(r, e) - lo) >> shift : dummy], 1u);
          }
      }
      uint32_t tau = lo;
      if (sample) {   // the same for the whole workgroup
        const uint32_t nsamp = block_sum(mine, sh, 0);
        const uint32_t need_s = (uint32_t)(((unsigned long long)2 * k * nsamp + n - 1) / n) + 8;
        int bs;
        uint32_t ab;
        find_bucket(sh, hsel, need_s, &bs, &ab);   // always: it also clears the next buffer
        if (need_s < nsamp && bs >= 0) tau = lo + ((uint32_t)bs << shift);
      }
      // candidates u >= tau.
      uint64_t cand[R];
      mine = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint64_t m = 0;
        if constexpr (R == 1) {
          for_slots(nvmax, [&](int e) { m |= (uint64_t)((e < nv[0]) & (reg[e] >= tau)) << e; });
        } else {
#pragma unroll kU
          for (int e = 0; e < kChunk; ++e) m |= (uint64_t)((e < nv[r]) & (key(r, e) >= tau)) << e;
        }
        cand[r] = m;
        mine += __builtin_popcountll(m);
      }
      ncand = sample ? block_sum(mine, sh, 1) : (uint32_t)n;   // without a sample every key is one
      if (ncand >= (uint32_t)k && ncand <= (uint32_t)kListCap) {
        // A thread's candidates take consecutive slots: one wave prefix sum of the counts and
        // one reservation per wave. With R = 1 the keys come from registers (unrolled, so the
        // register array is never indexed at run time); otherwise they are read again.
        if (t == 0) sh.list_n = 0;
        __syncthreads();
        const int incl = wave_inclusive_scan((int)mine);
        int base = 0;
        if (lane == 63 && incl) base = atomicAdd(&sh.list_n, incl);
        int slot = __builtin_amdgcn_readlane(base, 63) + incl - (int)mine;
        if constexpr (R == 1) {
          for_slots(nvmax, [&](int e) {
            if ((cand[0] >> e) & 1u) {
              sh.list_u[slot] = reg[e];
              sh.list_j[slot] = blk(0, e);
              ++slot;
            }
          });
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            uint64_t m = cand[r];
            while (m) {
              const int j = kChunk * (t + kSelThreads * r) + __builtin_ctzll(m);
              m &= m - 1;
              sh.list_u[slot] = score_key(s[j]);
              sh.list_j[slot] = j;
              ++slot;
            }
          }
        }
        __syncthreads();
        have_list = true;
        lo = tau;
      } else {
        // narrow over every key (branch-free: uncounted keys go to the lane's dummy bin).
        while (lo != hi) {
          shift = shift_for(lo, hi);
          const uint32_t clo = lo, span_all = hi - lo;
          if constexpr (R == 1) {
            for_slots(nvmax, [&](int e) {
              const uint32_t d = reg[e] - clo;
              atomicAdd(&sh.hbuf[hsel][((e < nv[0]) & (d <= span_all)) ? d >> shift : dummy], 1u);
            });
          } else {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll kU
              for (int e = 0; e < kChunk; ++e) {
                const uint32_t d = key(r, e) - clo;
                atomicAdd(&sh.hbuf[hsel][((e < nv[r]) & (d <= span_all)) ? d >> shift : dummy], 1u);
              }
          }
          __syncthreads();
          if (narrow_step(sh, hsel, shift, &lo, &hi, &need)) { all_of_bucket = true; break; }
        }
      }
    }
    if (!have_list) {  // masks from every key
      if constexpr (R == 1) {
        // slot e of wave w covers word w + 16e, bit = lane: one ballot each, one owner
        // (words of slots past the wave's last valid one stay as cleared at kernel start)
        const int wave = t >> 6;
        for_slots(nvmax, [&](int e) {
          const uint32_t u = reg[e];
          const bool ok = e < nv[0];
          const uint64_t bk = __ballot(ok & (all_of_bucket ? u >= lo : u > hi));
          const uint64_t bt = __ballot(ok & !all_of_bucket & (u == lo));
          if (lane == 0) { kept_w[wave + kSelWaves * e] = bk; tie_w[wave + kSelWaves * e] = bt; }
        });
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint64_t mk = 0, mt = 0;
#pragma unroll kU
          for (int e = 0; e < kChunk; ++e) {
            const uint32_t u = key(r, e);
            const bool ok = e < nv[r];
            mk |= (uint64_t)(ok & (all_of_bucket ? u >= lo : u > hi)) << e;
            mt |= (uint64_t)(ok & !all_of_bucket & (u == lo)) << e;
          }
          kept_w[t + kSelThreads * r] = mk;
          tie_w[t + kSelThreads * r] = mt;
        }
      }
      masks_done = true;
    }
  }
  if (have_list && !masks_done) {
    uint32_t llo = lo;
    narrow_list_and_mark<R, CAP>(sh, hsel, ncand, lo, hi, &need, &all_of_bucket, &llo, kept_w, tie_w);
    lo = llo;
  }
  __syncthreads();

  // The first `need` ties in block order join the kept set; then ascending ids. Each
  // thread reads and updates only its own words here, so no barrier is needed between.
  int sbuf = 0;   // block_exclusive_scan half
  if (!all_of_bucket) {
    int run = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = t + kSelThreads * r;
      const uint64_t m0 = tie_w[c];
      int tot;
      int before = run + block_exclusive_scan<kSelThreads>(__builtin_popcountll(m0), sh.scan, sbuf, &tot);
      uint64_t m = m0, take = 0;
      while (m && before < (int)need) {
        take |= m & (~m + 1);
        m &= m - 1;
        ++before;
      }
      kept_w[c] |= take;
      run += tot;
    }
  }
  int run = 0;
  if (R == 1 && n <= kStridedOut) {
    // Short request: the kept blocks sit in a few words, so instead of each word's owner
    // writing its ids one by one, thread t writes the ids of its blocks t + 1024*e, at the
    // word's prefix plus the kept bits below it in the word.
    const uint64_t m = kept_w[t];
    int tot;
    sh.wpre[t] = block_exclusive_scan<kSelThreads>(__builtin_popcountll(m), sh.scan, sbuf, &tot);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kStridedOut / kSelThreads; ++e) {
      const int j = t + kSelThreads * e;
      if (j < n) {
        const uint64_t w = kept_w[j >> 6];
        const uint64_t below = w & ((1ull << (j & 63)) - 1ull);
        if ((w >> (j & 63)) & 1ull) {
          const int pos = sh.wpre[j >> 6] + __builtin_popcountll(below);
          if (pos < k) out[pos] = j;
        }
      }
    }
    run = tot;
  } else {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = t + kSelThreads * r;
    uint64_t m = kept_w[c];
    int tot;
    int pos = run + block_exclusive_scan<kSelThreads>(__builtin_popcountll(m), sh.scan, sbuf, &tot);
    while (m) {
      const int j = kChunk * c + __builtin_ctzll(m);
      m &= m - 1;
      if (pos < k) out[pos] = j;
      ++pos;
    }
    run += tot;
  }
  }
  for (int i = run + t; i < k; i += kSelThreads) out[i] = -1;
  if (t == 0) sel_count[b] = min(run, k);
}

size_t topk_workspace_bytes(int B, int max_blocks) {
  (void)B;
  (void)max_blocks;
  return 0;
}

hipError_t launch_topk_select(const int32_t* scores, const int32_t* lens, const int32_t* page_max, int B,
                              int max_blocks, int max_pages, int k, int32_t* sel, int32_t* sel_count,
                              int T, hipStream_t stream) {
  const int chunks = (max_blocks + kChunk - 1) / kChunk;
  const int R = chunks <= kSelThreads ? 1 : chunks <= 2 * kSelThreads ? 2 : 4;
  // Many requests (prefill chunks): the R = 2 form with a 1,024-entry list (53 VGPRs, 78 KB of
  // LDS) fits two workgroups per CU where the R = 1 form (113 VGPRs, 119 KB) fits one; a
  // request whose candidates overflow the list takes the narrowing over all its keys instead.
  const bool many = B >= kManyRequests && R <= 2;
  const size_t lds = 2 * (size_t)kSelThreads * (many ? 2 : R) * sizeof(uint64_t);
  if (many)
    hipLaunchKernelGGL((topk_select_kernel<2, 1024>), dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       page_max, max_blocks, max_pages, k, sel, sel_count, T);
  else if (R == 1)
    hipLaunchKernelGGL(topk_select_kernel<1>, dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       page_max, max_blocks, max_pages, k, sel, sel_count, T);
  else if (R == 2)
    hipLaunchKernelGGL(topk_select_kernel<2>, dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       page_max, max_blocks, max_pages, k, sel, sel_count, T);
  else
    hipLaunchKernelGGL(topk_select_kernel<4>, dim3(B), dim3(kSelThreads), lds, stream, scores, lens,
                       page_max, max_blocks, max_pages, k, sel, sel_count, T);
  return hipGetLastError();
}

}  // namespace qsa
