// sparse_attn.hip - K3: paged gather of the kept tokens + bf16 GQA attention per slice.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes": the softmax and
// the value aggregation use the full (not pooled) K and V rows of the kept positions (second
// paragraph); under decode context parallelism a rank attends over one contiguous piece
// of the context (first paragraph and bullets). Slice p of request b covers the pages
// [p*S_b, (p+1)*S_b) with S_b = ceil(ceil(L_b/64)/P); its partial is
// (output normalised over the slice, lse = max + ln sum), or (0, -inf) when the slice
// holds no kept token.
//
// Work split. The kept blocks are ascending, so those of slice p form one run of
// sel_blocks. The run is cut into C shares of whole tiles (a tile = 4 kept blocks = 16
// tokens), and one workgroup of 4 waves (one per SIMD, so each wave owns a SIMD's whole
// register file) takes one share of one (request, slice, KV head). C is chosen on the host
// so that a launch has about kAttnTargetGroups workgroups. Each workgroup writes the
// partial of its share; the slice partial is the log-sum-exp merge of its C shares
// (slice_merge_kernel), the same formula that merges the slices.
//
// Inside a workgroup: every thread reads two kept slots (loaded together with sel_count and
// the length), counts (by wave ballots) the slots before and inside the slice and, for a
// slot inside, loads its physical page at once, so the only dependent global loads before
// the K/V rows are the ids and the page-table entries. The share's ids and the physical rows
// of their blocks' first tokens go to LDS; tiles are dealt round-robin to the waves;
// a wave issues the loads of up to kTilesInFlight tiles before it computes on the first,
// and keeps an online softmax over its tiles, two at a time where it has two. The 4 wave
// partials are merged in one LDS round, each thread finishing 8 output dims of one query head.
//
// Per wave and tile (lane = 16*q4 + i16):
//   K and V rows are loaded alike, 16 bytes per lane (lane: token 4*q4 + v of the tile, dims
//   8*i16 .. +7), so each load reads four whole 256-byte token rows.
//   S = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of K, reshaped from the
//   loaded rows through the wave's LDS area (lane: token i16, dims 32s + 8*q4 .. +7), B = 32
//   dims x 16 query heads of the KV head's group (rows past the group are zero). The result
//   gives lane (q4, i16) the scores of tokens 4*q4 .. 4*q4+3 (= kept block q4 of the tile) for
//   query head i16.
//   O^T += V^T P on v_mfma_f32_16x16x32_bf16, MFMA tile u (u = 0..7) taking dim 8*i16 + u as
//   its row i16, so the V rows need no transpose; the 32 k-slots are the lane's 8 tokens of
//   two tiles (or its 4 tokens twice), and P enters as a bf16 pair (hi, lo = p - hi), two
//   products with the same V operand, so the weights keep ~16 bits. A lane then ends up with
//   query head i16 and dims 32*q4 .. 32*q4+31 of the output, contiguous.
//   The dot products are exact bf16 products accumulated in fp32; softmax in fp32 (base-2
//   exponent with the scale folded in, the reference maximum moved only when a maximum grows
//   by more than 2^8).
// Absent tokens (past the share or at or past L_b) are not read: their lanes read row 0 of
// their own block again (present and finite), and their scores are -inf, so their weights
// are exactly 0 and no NaN row of a poisoned page can leak in.
#include <algorithm>

#include "qsa_device.h"

namespace qsa {

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kTilesInFlight = 4;        // tiles whose loads a wave issues before computing
constexpr int kPairTilesInFlight = 2;    // the same in the pair kernel (3 waves per SIMD)
constexpr int kPairAreaBytes = std::max(std::max(2 * 2 * kMaxK * 4, kAttnWaves * kMaxGroup * (kHeadDim + 4) * 4),
                                        kAttnWaves * 16 * 16 * 16);
constexpr int kAttnTargetGroups = 512;   // two workgroups per CU
constexpr int kMaxSplit = 32;            // shares per slice (tiny batches: one request, few heads)
constexpr int kPairMinTokens = 16;       // chunks of at least this many new tokens use the pair kernel
constexpr int kPairHeads = 4;            // at most this many KV heads per pair-kernel workgroup
constexpr int kPairMinGroups = 4096;     // ... as long as the launch keeps this many workgroups
static_assert(kMaxK <= 2 * kAttnThreads, "two kept slots per thread");

// Shares per slice for a launch of B requests, Hkv KV heads and P slices: the largest power
// of two <= min(kMaxSplit, ceil(kAttnTargetGroups / (B*Hkv*P))), at least 1.
int attn_split(int B, int Hkv, int P) {
  const long long base = (long long)B * Hkv * P;
  const long long want = std::min<long long>(kMaxSplit, (kAttnTargetGroups + base - 1) / base);
  int c = 1;
  while (2 * c <= want) c *= 2;
  return c;
}

// Two floats to a packed bf16 pair (lo in bits 0-15), round to nearest even, in one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

struct Tile {
  bf16x8 k[4];   // K rows as loaded: token 4*q4 + v, dims 8*i16 .. +7 (reshaped before use)
  u16x8 v[4];    // V rows: token 4*q4 + v, dims 8*i16 .. +7
  bool tv[4];    // token 4*q4 + v exists
  bool sv[4];    // (pair kernel) ... and is kept by the lane's column's new token
};

// Tile of 4 kept blocks starting at share slot bbase (share slots [0, nslot)); block ids and
// the physical rows of their first tokens (page * 64 + row, below 2^32 for any cache that fits
// in memory) come from LDS. kg and vg point at the lane's 16 bytes of row 0 of the caches
// (KV head g, dims 8*i16), rs is the row stride in elements: K and V are read alike, 256
// contiguous bytes per token row and 4 rows per load. A token past
// the share or at or past L (a poisoned or unrelated row) is not read: its lane loads row 0
// of its block instead (past the share, of the share's last block; always present, so
// finite), and the token is marked absent, which gives it a score of -inf and so a weight
// of exactly 0. Every lane loads, with
// no branch. PAIR: the lane's column belongs to new token tk of a pair, of length Lc <= L,
// which keeps a block of the share when bit tk of its s_mask entry is set.
template <bool PAIR>
__device__ __forceinline__ void load_tile(Tile& T, int bbase, int nslot, const int* s_sel, const uint32_t* s_ptok,
                                          const int* s_mask, int L, int Lc, int tk, const uint16_t* kg,
                                          const uint16_t* vg, uint32_t rs, int i16, int q4) {
  const int slot = bbase + q4, cs = min(slot, nslot - 1);
  const int blk = slot < nslot ? s_sel[cs] : -1;
  // Row 0 of the lane's block (of the share's last block past the share) always exists below
  // L; a token that is absent reads it again. One 64-bit product per tile, then 32-bit steps.
  const int nv = blk >= 0 ? L - 4 * blk : 0;     // the block's tokens below L (if > 3, all 4)
  const size_t off0 = (size_t)s_ptok[cs] * (2u * rs);
  const char* kp = reinterpret_cast<const char*>(kg) + off0;
  const char* vp = reinterpret_cast<const char*>(vg) + off0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    T.tv[v] = v < nv;
    const uint32_t d = T.tv[v] ? v * 2u * rs : 0u;
    T.k[v] = *reinterpret_cast<const bf16x8*>(kp + d);
    T.v[v] = *reinterpret_cast<const u16x8*>(vp + d);
  }
  if (PAIR) {
    const int nc = (blk >= 0 && ((s_mask[cs] >> tk) & 1)) ? Lc - 4 * blk : 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) T.sv[v] = v < nc;
  }
}

// The tile's K rows into the MFMA A layout (lane (i16, q4) of k-step s: token i16, dims
// 32s + 8*q4 .. +7) through the wave's 4 KiB LDS area: vector c (dims 8c .. 8c+7) of tile row
// r (token 4*(r/4) + r%4 of the tile) at r * 16 + (c ^ r), so that the 16 rows a lane group
// writes or reads at once fall in different banks. One wave's LDS operations run in order, so
// a later tile's writes follow this tile's reads.
__device__ __forceinline__ void k_operands(const Tile& T, bf16x8* area, int i16, int q4, bf16x8 (&ka)[4]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int r = 4 * q4 + v;
    area[r * 16 + (i16 ^ r)] = T.k[v];
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) ka[s] = area[i16 * 16 + ((4 * s + q4) ^ i16)];
}

constexpr float kRescaleSlack = 8.f;   // log2 of the largest weight summed against a stale maximum

// One tile into the wave's online softmax state (m_run, l_run in base-2 units; acc = O^T).
template <bool PAIR>
__device__ __forceinline__ void attend_tile(const Tile& T, const bf16x8* qa, float scale_log2, float& m_run,
                                            float& l_run, f32x4* acc, bf16x8* karea, int i16, int q4) {
  bf16x8 ka[4];
  k_operands(T, karea, i16, q4, ka);
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qa[s], sc, 0, 0, 0);

  float sv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) sv[v] = (PAIR ? T.sv[v] : T.tv[v]) ? sc[v] * scale_log2 : -INFINITY;
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  // The reference maximum moves only when some lane's tile maximum exceeds it by more than
  // kRescaleSlack (a wave-uniform branch); until then weights up to 2^kRescaleSlack are summed
  // against the old reference, which the final division by l_run cancels (l_run and acc share
  // it), so the state is rescaled about once per share instead of whenever a maximum moves.
  if (__ballot(mt > m_run + kRescaleSlack)) {
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  // p = 2^(s - m) <= 2^kRescaleSlack on v_exp_f32; P enters the PV product as a bf16 pair (hi = bf16(p),
  // lo = bf16(p - hi)), so the weights keep ~16 bits.
  float pv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) pv[v] = __builtin_amdgcn_exp2f(sv[v] - m_use);
  l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
  union { uint32_t w[4]; bf16x8 v; } bp;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    bp.w[i] = cvt_bf16x2(pv[2 * i], pv[2 * i + 1]);
    bp.w[2 + i] = cvt_bf16x2(pv[2 * i] - __uint_as_float(bp.w[i] << 16),
                             pv[2 * i + 1] - __uint_as_float(bp.w[i] & 0xFFFF0000u));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    union { uint32_t w[4]; bf16x8 v; } va;
    va.w[0] = pack2(T.v[0][u], T.v[1][u]);
    va.w[1] = pack2(T.v[2][u], T.v[3][u]);
    va.w[2] = va.w[0];
    va.w[3] = va.w[1];
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, bp.v, acc[u], 0, 0, 0);
  }
}

// Two tiles at once: one softmax update over their 32 tokens (one maximum, one rescale), and
// the PV product with the lane's 8 distinct tokens (its 4 of tile A, then its 4 of tile B) on
// the 32 k-slots, hi and lo parts of P as two products with the same V operand, so V needs
// no duplication.
template <bool PAIR>
__device__ __forceinline__ void attend_two(const Tile& A, const Tile& B, const bf16x8* qa, float scale_log2,
                                           float& m_run, float& l_run, f32x4* acc, bf16x8* karea, int i16, int q4) {
  bf16x8 ka[4], kb[4];
  k_operands(A, karea, i16, q4, ka);
  k_operands(B, karea, i16, q4, kb);
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qa[s], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[s], qa[s], sb, 0, 0, 0);
  }
  float sv[8];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    sv[v] = (PAIR ? A.sv[v] : A.tv[v]) ? sa[v] * scale_log2 : -INFINITY;
    sv[4 + v] = (PAIR ? B.sv[v] : B.tv[v]) ? sb[v] * scale_log2 : -INFINITY;
  }
  float mt = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  if (__ballot(mt > m_run + kRescaleSlack)) {   // as in attend_tile
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] *= alpha;
    m_run = m_new;
  }
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float pv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(sv[e] - m_use);
  l_run += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
  union { uint32_t w[4]; bf16x8 v; } ph, pl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ph.w[i] = cvt_bf16x2(pv[2 * i], pv[2 * i + 1]);
    pl.w[i] = cvt_bf16x2(pv[2 * i] - __uint_as_float(ph.w[i] << 16),
                         pv[2 * i + 1] - __uint_as_float(ph.w[i] & 0xFFFF0000u));
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    union { uint32_t w[4]; bf16x8 v; } va;
    va.w[0] = pack2(A.v[0][u], A.v[1][u]);
    va.w[1] = pack2(A.v[2][u], A.v[3][u]);
    va.w[2] = pack2(B.v[0][u], B.v[1][u]);
    va.w[3] = pack2(B.v[2][u], B.v[3][u]);
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, ph.v, acc[u], 0, 0, 0);
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, pl.v, acc[u], 0, 0, 0);
  }
}

// Grid (C * Hkv * T, P, B_req): blockIdx.x = (t * Hkv + g) * C + c for new token t of request
// b_req = blockIdx.z, slice p = blockIdx.y, and b = b_req*T + t is the virtual request
// (page-table row b_req, length L - (T-1-t)). With many new tokens (a prefill chunk) the
// workgroups of one (request, slice) are dispatched together, so the slice's K/V rows, kept
// by several tokens each, are re-read while they sit in the 256 MB MALL instead of again from
// HBM. With T = 1 it is the single-token grid (C * Hkv, P, B). Writes the partial of share c of
// (b, p, KV head g) for the query heads of g: sub_out [B, P, C, Hq, 128] (normalised over the share), sub_lse [B, P, C, Hq]
// (natural log; -inf for an empty share, whose output is 0).
__global__ __launch_bounds__(kAttnThreads, 2) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int Hq, int Hkv,
    int max_pages, int k, int P, int C, int T, float scale_log2, float* __restrict__ sub_out,
    float* __restrict__ sub_lse) {
  const int gc = blockIdx.x % (C * Hkv), tq = blockIdx.x / (C * Hkv);
  const int g = gc / C, c = gc - g * C, p = blockIdx.y, b = blockIdx.z * T + tq;
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int group = Hq / Hkv;
  const int32_t* sb = sel + (size_t)b * k;
  // Kept slots t and t + 256 are loaded first, whether or not the slot is below K (every
  // slot < k is in bounds), so the loads wait neither for sel_count nor for the length.
  int jraw[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int slot = t + kAttnThreads * r;
    jraw[r] = slot < k ? sb[slot] : 0;
  }
  const int L = draft_length(lens, b, T);
  const int K = sel_count[b];
  const int32_t* ptab = page_table + (size_t)(b / T) * max_pages;
  const size_t share = ((size_t)b * P + p) * C + c;

  __shared__ int s_cnt[kAttnWaves][2];
  __shared__ int s_sel[kMaxK];      // kept block ids of the share
  __shared__ uint32_t s_ptok[kMaxK];   // and the physical rows of their first tokens
  __shared__ float s_m[kAttnWaves][kMaxGroup];
  __shared__ float s_l[kAttnWaves][kMaxGroup];
  __shared__ float s_o[kAttnWaves][kMaxGroup][kHeadDim + 4];
  __shared__ bf16x8 s_kr[kAttnWaves][16 * 16];   // each wave's K reshaping area (k_operands)

  const int npages = (L + kPageSize - 1) / kPageSize;
  const int S = (npages + P - 1) / P;
  const int pg0 = min(p * S, npages), pg1 = min((p + 1) * S, npages);

  // Kept slots t and t + 256: block id, position relative to the slice, physical row of the
  // block's first token if inside.
  int jr[2];
  uint32_t pr[2];
  bool inr[2];
  int nbefore = 0, ninside = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int slot = t + kAttnThreads * r;
    const bool valid = slot < K;
    const int j = valid ? jraw[r] : 0;
    const int pg = j / kBlocksPerPage;
    inr[r] = valid && pg >= pg0 && pg < pg1;
    jr[r] = j;
    pr[r] = inr[r] ? (uint32_t)ptab[pg] * kPageSize + kTokensPerBlock * (j % kBlocksPerPage) : 0u;
    nbefore += __builtin_popcountll(__ballot(valid && pg < pg0));
    ninside += __builtin_popcountll(__ballot(inr[r]));
  }
  if (lane == 0) { s_cnt[wave][0] = nbefore; s_cnt[wave][1] = ninside; }
  // Q operand: query head i16 of this KV head's group, dims 32s + 8*q4 .. +7.
  bf16x8 qa[4];
  if (i16 < group) {
    const uint16_t* qrow = q + ((size_t)b * Hq + (size_t)g * group + i16) * kHeadDim + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = bf16x8{};
  }
  __syncthreads();
  int seg0 = 0, nin = 0;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) { seg0 += s_cnt[w][0]; nin += s_cnt[w][1]; }
  const int ntiles = (nin + 3) / 4;
  const int tps = (ntiles + C - 1) / C;            // tiles per share
  const int tile0 = min(c * tps, ntiles), nt = min(tile0 + tps, ntiles) - tile0;
  const int slot0 = 4 * tile0, nslot = min(4 * (tile0 + nt), nin) - slot0;

  if (nt == 0) {   // empty share (the same for the whole workgroup)
    for (int i = t; i < group * 32; i += kAttnThreads) {
      const int h = i >> 5, d4 = i & 31;
      *reinterpret_cast<f32x4*>(sub_out + (share * Hq + (size_t)g * group + h) * kHeadDim + 4 * d4) =
          f32x4{0.f, 0.f, 0.f, 0.f};
      if (d4 == 0) sub_lse[share * Hq + (size_t)g * group + h] = -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int ls = t + kAttnThreads * r - seg0 - slot0;
    if (inr[r] && ls >= 0 && ls < nslot) { s_sel[ls] = jr[r]; s_ptok[ls] = pr[r]; }
  }
  __syncthreads();

  const uint16_t* kg = kc + (size_t)g * kHeadDim + 8 * i16;
  const uint16_t* vg = vc + (size_t)g * kHeadDim + 8 * i16;
  const uint32_t rs = (uint32_t)Hkv * kHeadDim;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int r0 = wave; r0 < nt; r0 += kAttnWaves * kTilesInFlight) {
    Tile T[kTilesInFlight];
#pragma unroll
    for (int m = 0; m < kTilesInFlight; ++m) {
      const int ti = r0 + kAttnWaves * m;
      if (ti < nt) load_tile<false>(T[m], 4 * ti, nslot, s_sel, s_ptok, nullptr, L, L, 0, kg, vg, rs, i16, q4);
    }
#pragma unroll
    for (int m = 0; m < kTilesInFlight; m += 2) {
      const int ti = r0 + kAttnWaves * m;
      if (ti + kAttnWaves < nt) attend_two<false>(T[m], T[m + 1], qa, scale_log2, m_run, l_run, acc, s_kr[wave], i16, q4);
      else if (ti < nt) attend_tile<false>(T[m], qa, scale_log2, m_run, l_run, acc, s_kr[wave], i16, q4);
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  // Merge of the 4 wave partials: lane (q4, i16) holds head i16 and dims 8*(4*q4 + r) + u
  // in acc[u][r]; afterwards thread t finishes head t/16, dims 8*(t%16) .. +7.
  if (q4 == 0) { s_m[wave][i16] = m_run; s_l[wave][i16] = l_tot; }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][i16][8 * (4 * q4 + r) + u] = acc[u][r];
  __syncthreads();
  const int h = t >> 4, d0 = 8 * (t & 15);
  if (h < group) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float f = exp2f(s_m[w][h] - Mu);
      l += s_l[w][h] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += s_o[w][h][d0 + e] * f;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = sub_out + (share * Hq + (size_t)g * group + h) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    if (d0 == 0)
      sub_lse[share * Hq + (size_t)g * group + h] =
          l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// Exclusive prefix sum of one value per thread over the workgroup, with the total in *tot.
// Every thread must reach it; s_tmp holds kAttnWaves ints.
__device__ __forceinline__ int block_scan(int x, int* s_tmp, int* tot) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(x);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) {
    const int v = s_tmp[w];
    before += w < wave ? v : 0;
    all += v;
  }
  __syncthreads();
  *tot = all;
  return before + inc - x;
}

// Number of entries of the ascending array a[0, n) below v.
__device__ __forceinline__ int lower_bound_lds(const int* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// Chunks of new tokens with 8 query heads per KV head: new tokens 2m and 2m+1 of a request
// (virtual requests b*T + 2m and b*T + 2m + 1) share one workgroup per (slice, share, group of
// hpw KV heads). The 16 MFMA columns of the single-token kernel, half of them empty at a group of 8, hold
// the two tokens' heads (column i16: token i16/8, head i16%8), and the kernel gathers the
// union of the two tokens' kept blocks inside the slice once: each block is marked with the
// tokens that keep it, and a column's scores are -inf on the blocks its token does not keep
// or past its length. A block kept by both tokens is read once instead of twice; with
// unrelated selections the union is the two lists side by side and the work is the same as
// two single-token workgroups'. Each token's slice is its own (its page count can differ by
// one from its neighbour's). The share partials written are exactly the single-token
// kernel's, per virtual request. The union, its rows and masks are built once for the hpw KV
// heads (1, 2 or 4): 4/hpw waves per head split the tiles and merge through LDS, or with one
// wave per head the wave writes its head's partial from its registers. Grid
// (C * (Hkv/hpw) * ceil(T/2), P, B_req). Three workgroups per CU (three waves per SIMD): a
// wave loads kPairTilesInFlight tiles ahead, and one LDS area serves the union build, the K
// reshaping and the final merge in turn.
__global__ __launch_bounds__(kAttnThreads, 3) void sparse_attn_pair_kernel(   // 3 waves per SIMD
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int Hq, int Hkv,
    int max_pages, int k, int P, int C, int T, int hpw, float scale_log2, float* __restrict__ sub_out,
    float* __restrict__ sub_lse) {
  constexpr int G = 8;   // query heads per KV head
  const int HG = Hkv / hpw;   // KV-head groups; this workgroup takes heads g0 .. g0+hpw-1
  const int gc = blockIdx.x % (C * HG), m = blockIdx.x / (C * HG);
  const int g0 = (gc / C) * hpw, c = gc % C, p = blockIdx.y, breq = blockIdx.z;
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int ntok = min(2, T - 2 * m);   // 1 for the last token of an odd chunk
  const int vr0 = breq * T + 2 * m;
  int jraw[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int slot = t + kAttnThreads * r;
      jraw[i][r] = i < ntok && slot < k ? sel[(size_t)(vr0 + i) * k + slot] : 0;
    }
  int Lt[2], Kt[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    Lt[i] = i < ntok ? draft_length(lens, vr0 + i, T) : 0;
    Kt[i] = i < ntok ? sel_count[vr0 + i] : 0;
  }
  const int32_t* ptab = page_table + (size_t)breq * max_pages;

  __shared__ int s_cnt[kAttnWaves][2][2];
  __shared__ int s_tmp[kAttnWaves];
  __shared__ int s_sel[2 * kMaxK];      // the share's part of the union of the two runs
  __shared__ uint32_t s_ptok[2 * kMaxK];
  __shared__ int s_mask[2 * kMaxK];     // bit i: token i keeps the block
  __shared__ float s_m[kAttnWaves][kMaxGroup];
  __shared__ float s_l[kAttnWaves][kMaxGroup];
  // One area for three uses that a barrier separates: each token's run while the union is
  // built, the waves' K reshaping areas in the tile loop, the wave partials in the final
  // merge. Sharing it keeps the workgroup at 47 KB of LDS, so three fit on a CU.
  __shared__ __attribute__((aligned(16))) unsigned char s_area[kPairAreaBytes];
  int (*s_run)[kMaxK] = reinterpret_cast<int (*)[kMaxK]>(s_area);            // kept ids in slice p
  uint32_t (*s_runp)[kMaxK] = reinterpret_cast<uint32_t (*)[kMaxK]>(s_area + 2 * kMaxK * 4);  // their rows
  bf16x8 (*s_kr)[16 * 16] = reinterpret_cast<bf16x8 (*)[16 * 16]>(s_area);
  float (*s_o)[kMaxGroup][kHeadDim + 4] = reinterpret_cast<float (*)[kMaxGroup][kHeadDim + 4]>(s_area);

  int jr[2][2];
  uint32_t pr[2][2];
  bool inr[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int npages = (Lt[i] + kPageSize - 1) / kPageSize;
    const int S = (npages + P - 1) / P;
    const int pg0 = min(p * S, npages), pg1 = min((p + 1) * S, npages);
    int nbefore = 0, ninside = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int slot = t + kAttnThreads * r;
      const bool valid = slot < Kt[i];
      const int j = valid ? jraw[i][r] : 0;
      const int pg = j / kBlocksPerPage;
      inr[i][r] = valid && pg >= pg0 && pg < pg1;
      jr[i][r] = j;
      pr[i][r] = inr[i][r] ? (uint32_t)ptab[pg] * kPageSize + kTokensPerBlock * (j % kBlocksPerPage) : 0u;
      nbefore += __builtin_popcountll(__ballot(valid && pg < pg0));
      ninside += __builtin_popcountll(__ballot(inr[i][r]));
    }
    if (lane == 0) { s_cnt[wave][i][0] = nbefore; s_cnt[wave][i][1] = ninside; }
  }
  const int tk = i16 >> 3;   // the lane's column belongs to new token tk
  __syncthreads();
  int seg0[2] = {0, 0}, nin[2] = {0, 0};
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w)
#pragma unroll
    for (int i = 0; i < 2; ++i) { seg0[i] += s_cnt[w][i][0]; nin[i] += s_cnt[w][i][1]; }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ls = t + kAttnThreads * r - seg0[i];
      if (inr[i][r]) { s_run[i][ls] = jr[i][r]; s_runp[i][ls] = pr[i][r]; }
    }
  __syncthreads();

  // Union of the two ascending runs. Entry ls of run i lands at ls + (number of entries of
  // the other run below it) - (number of entries before it that both runs hold); an entry of
  // run 1 that run 0 also holds is not placed again (run 0's copy carries both bits).
  int lb[2][2];
  bool both[2][2];
  int pref[2][2], nboth = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int run_tot = 0;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ls = t + kAttnThreads * r;
      lb[i][r] = 0;
      both[i][r] = false;
      if (ls < nin[i]) {
        const int id = s_run[i][ls];
        lb[i][r] = lower_bound_lds(s_run[1 - i], nin[1 - i], id);
        both[i][r] = lb[i][r] < nin[1 - i] && s_run[1 - i][lb[i][r]] == id;
      }
      int tot;
      pref[i][r] = run_tot + block_scan(both[i][r] ? 1 : 0, s_tmp, &tot);
      run_tot += tot;
    }
    if (i == 0) nboth = run_tot;
  }
  const int nU = nin[0] + nin[1] - nboth;
  const int ntiles = (nU + 3) / 4;
  const int tps = (ntiles + C - 1) / C;            // tiles per share
  const int tile0 = min(c * tps, ntiles), nt = min(tile0 + tps, ntiles) - tile0;
  const int slot0 = 4 * tile0, nslot = min(4 * (tile0 + nt), nU) - slot0;

  if (nt == 0) {   // empty share for both tokens, every head of the workgroup
    for (int i = t; i < ntok * hpw * G * 32; i += kAttnThreads) {
      const int tt = i / (hpw * G * 32), hh = (i >> 5) % (hpw * G), d4 = i & 31;
      const size_t share = ((size_t)(vr0 + tt) * P + p) * C + c;
      *reinterpret_cast<f32x4*>(sub_out + (share * Hq + (size_t)g0 * G + hh) * kHeadDim + 4 * d4) =
          f32x4{0.f, 0.f, 0.f, 0.f};
      if (d4 == 0) sub_lse[share * Hq + (size_t)g0 * G + hh] = -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int ls = t + kAttnThreads * r;
      if (ls < nin[i] && !(i == 1 && both[i][r])) {
        const int u = ls + lb[i][r] - pref[i][r] - slot0;
        if (u >= 0 && u < nslot) {
          s_sel[u] = s_run[i][ls];
          s_ptok[u] = s_runp[i][ls];
          s_mask[u] = i == 0 ? (both[i][r] ? 3 : 1) : 2;
        }
      }
    }
  __syncthreads();

  const uint32_t rs = (uint32_t)Hkv * kHeadDim;
  const int Lmax = max(Lt[0], Lt[1]), Lc = Lt[tk];
  // The union, its rows and masks serve the workgroup's hpw KV heads at once: wph = 4/hpw waves
  // per head, wave `wave` on head g0 + wave/wph, taking every wph-th tile of the share.
  const int wph = kAttnWaves / hpw, g = g0 + wave / wph, sub = wave % wph;
  // Q operand: column i16 = head g*8 + i16%8 of new token tk, dims 32s + 8*q4 .. +7.
  bf16x8 qa[4];
  if (tk < ntok) {
    const uint16_t* qrow = q + ((size_t)(vr0 + tk) * Hq + (size_t)g * G + (i16 & 7)) * kHeadDim + 8 * q4;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = bf16x8{};
  }
  const uint16_t* kg = kc + (size_t)g * kHeadDim + 8 * i16;
  const uint16_t* vg = vc + (size_t)g * kHeadDim + 8 * i16;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = sub; r0 < nt; r0 += wph * kPairTilesInFlight) {
    Tile Ts[kPairTilesInFlight];
#pragma unroll
    for (int mm = 0; mm < kPairTilesInFlight; ++mm) {
      const int ti = r0 + wph * mm;
      if (ti < nt)
        load_tile<true>(Ts[mm], 4 * ti, nslot, s_sel, s_ptok, s_mask, Lmax, Lc, tk, kg, vg, rs, i16, q4);
    }
#pragma unroll
    for (int mm = 0; mm < kPairTilesInFlight; mm += 2) {
      const int ti = r0 + wph * mm;
      if (ti + wph < nt) attend_two<true>(Ts[mm], Ts[mm + 1], qa, scale_log2, m_run, l_run, acc, s_kr[wave], i16, q4);
      else if (ti < nt) attend_tile<true>(Ts[mm], qa, scale_log2, m_run, l_run, acc, s_kr[wave], i16, q4);
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  if (wph == 1) {
    // The wave holds its head's whole share: lane (q4, i16) writes column i16's dims
    // 8*(4*q4 + r) .. +7 from acc[0..7][r], normalised, and lanes q4 = 0 the lse.
    if (tk < ntok) {
      const size_t share = ((size_t)(vr0 + tk) * P + p) * C + c;
      const int hg = g * G + (i16 & 7);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* dst = sub_out + (share * Hq + hg) * kHeadDim + 32 * q4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<f32x4*>(dst + 8 * r) =
            f32x4{acc[0][r] * inv, acc[1][r] * inv, acc[2][r] * inv, acc[3][r] * inv};
        *reinterpret_cast<f32x4*>(dst + 8 * r + 4) =
            f32x4{acc[4][r] * inv, acc[5][r] * inv, acc[6][r] * inv, acc[7][r] * inv};
      }
      if (q4 == 0)
        sub_lse[share * Hq + hg] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    }
    return;
  }
  // Several waves per head: their partials merge through LDS, as in the single-token kernel,
  // once every wave is done with its reshaping area (the same LDS).
  __syncthreads();
  if (q4 == 0) { s_m[wave][i16] = m_run; s_l[wave][i16] = l_tot; }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][i16][8 * (4 * q4 + r) + u] = acc[u][r];
  __syncthreads();
  for (int it = t; it < hpw * 16 * 16; it += kAttnThreads) {   // (head of the group, column, 8 dims)
    const int gi = it >> 8, h = (it >> 4) & 15, d0 = 8 * (it & 15), th = h >> 3;
    if (th >= ntok) continue;
    const int w0 = gi * wph;
    float M = -INFINITY;
    for (int w = w0; w < w0 + wph; ++w) M = fmaxf(M, s_m[w][h]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int w = w0; w < w0 + wph; ++w) {
      const float f = exp2f(s_m[w][h] - Mu);
      l += s_l[w][h] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += s_o[w][h][d0 + e] * f;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const size_t share = ((size_t)(vr0 + th) * P + p) * C + c;
    const int hg = (g0 + gi) * G + (h & 7);
    float* dst = sub_out + (share * Hq + hg) * kHeadDim + d0;
    *reinterpret_cast<f32x4*>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    if (d0 == 0)
      sub_lse[share * Hq + hg] = l > 0.f ? (M + __log2f(l)) * 0.69314718055994531f : -INFINITY;
  }
}

size_t attn_sub_out_bytes(int B, int Hq, int Hkv, int P) {
  return align256((size_t)B * P * attn_split(B, Hkv, P) * Hq * kHeadDim * sizeof(float));
}

// One share per slice needs no workspace: the attention kernel writes the slice partials.
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int P) {
  if (attn_split(B, Hkv, P) == 1) return 0;
  return attn_sub_out_bytes(B, Hq, Hkv, P) +
         align256((size_t)B * P * attn_split(B, Hkv, P) * Hq * sizeof(float));
}

hipError_t launch_slice_merge(const float* so, const float* sl, int B, int P, int C, int Hq, float* part_out,
                              float* part_lse, float* out, float* out_lse, hipStream_t stream);
// Several shares per slice: their partials go to the workspace, and slice_merge_kernel then
// writes the slice partials and, when out != NULL, the merge of the slices. One share per
// slice (a share partial is then the slice partial, bit for bit): the attention kernel writes
// the slice partials itself and, when out != NULL, the same merge kernel reads them in place
// and writes only the merged result.
hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* page_table,
                              const int32_t* lens, const int32_t* sel, const int32_t* sel_count, int B,
                              int Hq, int Hkv, int max_pages, int k, int P, float scale,
                              float* part_out, float* part_lse, float* out, float* out_lse,
                              void* workspace, int T, hipStream_t stream) {
  const int C = attn_split(B, Hkv, P);
  float* sub_out = C == 1 ? part_out : static_cast<float*>(workspace);
  float* sub_lse = C == 1 ? part_lse
                          : reinterpret_cast<float*>(static_cast<char*>(workspace) + attn_sub_out_bytes(B, Hq, Hkv, P));
  const float scale_log2 = scale * 1.4426950408889634f;
  if ((long long)C * Hkv * T > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (T >= kPairMinTokens && Hq == 8 * Hkv) {
    // KV heads per workgroup: 4 or 2 when it divides Hkv and still leaves kPairMinGroups
    // workgroups (fewer, larger workgroups share the union's setup but need enough of them in
    // flight), else 1.
    const long long per_head = (long long)C * ((T + 1) / 2) * P * (B / T);
    int hpw = 1;
    for (int h = kPairHeads; h > 1; h /= 2)   // 4 or 2 (the 4 waves split evenly over the heads)
      if (Hkv % h == 0 && per_head * (Hkv / h) >= kPairMinGroups) { hpw = h; break; }
    hipLaunchKernelGGL(sparse_attn_pair_kernel, dim3(C * (Hkv / hpw) * ((T + 1) / 2), P, B / T),
                       dim3(kAttnThreads), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc), page_table, lens, sel,
                       sel_count, Hq, Hkv, max_pages, k, P, C, T, hpw, scale_log2, sub_out, sub_lse);
  } else {
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(C * Hkv * T, P, B / T), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), page_table, lens, sel, sel_count, Hq, Hkv,
                     max_pages, k, P, C, T, scale_log2, sub_out, sub_lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (C == 1)
    return out != nullptr ? launch_slice_merge(part_out, part_lse, B, P, 1, Hq, nullptr, nullptr, out, out_lse, stream)
                          : e;
  return launch_slice_merge(sub_out, sub_lse, B, P, C, Hq, part_out, part_lse, out, out_lse, stream);
}

}  // namespace qsa
