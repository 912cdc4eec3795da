// sparse_attn.hip - K3: paged gather of the kept tokens + bf16 GQA attention per slice.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes": the softmax and
// the value aggregation run on the uncompressed K and V of the kept positions (second
// paragraph), and each decode-context-parallel rank reads only its slice of the context
// (first paragraph and bullets). Slice p of request b covers the pages
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
// the K/V rows are the ids and the page-table entries. The share's ids and pages go to LDS; tiles are dealt round-robin to the waves;
// a wave issues the loads of up to kTilesInFlight tiles before it computes on the first,
// and keeps an online softmax over its tiles. The 4 wave partials are merged in one LDS
// round, each thread finishing 8 output dims of one query head.
//
// Per wave and tile (lane = 16*q4 + i16):
//   S = K Q^T on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 dims of K, loaded straight
//   from the paged cache (lane: token i16, dims 32s + 8*q4 .. +7), B = 32 dims x 16
//   query heads of the KV head's group (rows past the group are zero). The result gives
//   lane (q4, i16) the scores of tokens 4*q4 .. 4*q4+3 (= kept block q4 of the tile) for
//   query head i16.
//   O^T += V^T P on v_mfma_f32_16x16x32_bf16 with k = 32 slots = the lane's 4 tokens
//   twice: P enters as a bf16 pair (hi, lo = p - hi), so the weights keep ~16 bits;
//   V rows are loaded 16 bytes per lane (lane: token 4*q4+v, dims 8*i16 .. +7) and
//   MFMA tile u (u = 0..7) takes dim 8*i16 + u as its row i16. A lane then ends up with
//   query head i16 and dims 32*q4 .. 32*q4+31 of the output, contiguous.
//   The dot products are exact bf16 products accumulated in fp32; softmax in fp32
//   (base-2 exponent with the scale folded in).
// Masked tokens (past the share or past L_b) are never loaded: their K and V registers
// stay zero and their scores are -inf, so NaN rows cannot leak in.
#include <algorithm>

#include "qsa_device.h"

namespace qsa {

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * 64;
constexpr int kTilesInFlight = 4;        // tiles whose loads a wave issues before computing
constexpr int kAttnTargetGroups = 512;   // two workgroups per CU
constexpr int kMaxSplit = 32;            // shares per slice (tiny batches: one request, few heads)
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

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;  // finite inputs only (here 0 <= f <= 1)
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return (lo16 & 0xFFFFu) | (hi16 << 16); }

struct Tile {
  bf16x8 k[4];   // K operand: token i16, dims 32s + 8*q4 .. +7
  u16x8 v[4];    // V rows: token 4*q4 + v, dims 8*i16 .. +7
  bool tv[4];    // token 4*q4 + v exists
};

// Tile of 4 kept blocks starting at share slot bbase (share slots [0, nslot)); block ids and
// their page ids come from LDS.
__device__ __forceinline__ void load_tile(Tile& T, int bbase, int nslot, const int* s_sel, const int* s_page,
                                          int L, const uint16_t* kc, const uint16_t* vc, int Hkv, int g,
                                          int i16, int q4) {
  {
    const int slot = bbase + (i16 >> 2);
    const int tok = slot < nslot ? 4 * s_sel[slot] + (i16 & 3) : L;
    if (tok < L) {
      const int page = s_page[slot];
      const uint16_t* krow = kc + (((size_t)page * kPageSize + (tok & 63)) * Hkv + g) * kHeadDim + 8 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) T.k[s] = *reinterpret_cast<const bf16x8*>(krow + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) T.k[s] = bf16x8{};
    }
  }
  const int slot = bbase + q4;
  const int blk = slot < nslot ? s_sel[slot] : -1;
  const int page = blk >= 0 ? s_page[slot] : 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tok = 4 * blk + v;
    T.tv[v] = blk >= 0 && tok < L;
    if (T.tv[v]) {
      const uint16_t* vrow = vc + (((size_t)page * kPageSize + (tok & 63)) * Hkv + g) * kHeadDim + 8 * i16;
      T.v[v] = *reinterpret_cast<const u16x8*>(vrow);
    } else {
      T.v[v] = u16x8{};
    }
  }
}

// One tile into the wave's online softmax state (m_run, l_run in base-2 units; acc = O^T).
__device__ __forceinline__ void attend_tile(const Tile& T, const bf16x8* qa, float scale_log2, float& m_run,
                                            float& l_run, f32x4* acc) {
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(T.k[s], qa[s], sc, 0, 0, 0);

  float sv[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) sv[v] = T.tv[v] ? sc[v] * scale_log2 : -INFINITY;
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
  mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
  const float m_new = fmaxf(m_run, mt);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2f(m_run - m_use);
  float pv[4];
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    pv[v] = exp2f(sv[v] - m_use);
    ph[v] = bf16_bits_rne(pv[v]);
    pl[v] = bf16_bits_rne(pv[v] - __uint_as_float(ph[v] << 16));
  }
  l_run = l_run * alpha + (pv[0] + pv[1]) + (pv[2] + pv[3]);
  m_run = m_new;

  union { uint32_t w[4]; bf16x8 v; } bp;
  bp.w[0] = pack2(ph[0], ph[1]);
  bp.w[1] = pack2(ph[2], ph[3]);
  bp.w[2] = pack2(pl[0], pl[1]);
  bp.w[3] = pack2(pl[2], pl[3]);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    acc[u] *= alpha;
    union { uint32_t w[4]; bf16x8 v; } va;
    va.w[0] = pack2(T.v[0][u], T.v[1][u]);
    va.w[1] = pack2(T.v[2][u], T.v[3][u]);
    va.w[2] = va.w[0];
    va.w[3] = va.w[1];
    acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, bp.v, acc[u], 0, 0, 0);
  }
}

// Grid (C * Hkv, P, B). With T draft tokens per request, b is the virtual request
// b_req*T + t (page-table row b_req, length L - (T-1-t)). Writes the partial of share c of
// (b, p, KV head g) for the query heads of g: sub_out [B, P, C, Hq, 128] (normalised over the share), sub_lse [B, P, C, Hq]
// (natural log; -inf for an empty share, whose output is 0).
__global__ __launch_bounds__(kAttnThreads) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int Hq, int Hkv,
    int max_pages, int k, int P, int C, int T, float scale_log2, float* __restrict__ sub_out,
    float* __restrict__ sub_lse) {
  const int g = blockIdx.x / C, c = blockIdx.x - g * C, p = blockIdx.y, b = blockIdx.z;
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
  __shared__ int s_page[kMaxK];     // and their physical pages
  __shared__ float s_m[kAttnWaves][kMaxGroup];
  __shared__ float s_l[kAttnWaves][kMaxGroup];
  __shared__ float s_o[kAttnWaves][kMaxGroup][kHeadDim + 4];

  const int npages = (L + kPageSize - 1) / kPageSize;
  const int S = (npages + P - 1) / P;
  const int pg0 = min(p * S, npages), pg1 = min((p + 1) * S, npages);

  // Kept slots t and t + 256: block id, position relative to the slice, page if inside.
  int jr[2], pr[2];
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
    pr[r] = inr[r] ? ptab[pg] : 0;
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
    if (inr[r] && ls >= 0 && ls < nslot) { s_sel[ls] = jr[r]; s_page[ls] = pr[r]; }
  }
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int r0 = wave; r0 < nt; r0 += kAttnWaves * kTilesInFlight) {
    Tile T[kTilesInFlight];
#pragma unroll
    for (int m = 0; m < kTilesInFlight; ++m) {
      const int ti = r0 + kAttnWaves * m;
      if (ti < nt) load_tile(T[m], 4 * ti, nslot, s_sel, s_page, L, kc, vc, Hkv, g, i16, q4);
    }
#pragma unroll
    for (int m = 0; m < kTilesInFlight; ++m) {
      const int ti = r0 + kAttnWaves * m;
      if (ti < nt) attend_tile(T[m], qa, scale_log2, m_run, l_run, acc);
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

size_t attn_sub_out_bytes(int B, int Hq, int Hkv, int P) {
  return align256((size_t)B * P * attn_split(B, Hkv, P) * Hq * kHeadDim * sizeof(float));
}

size_t attn_workspace_bytes(int B, int Hq, int Hkv, int P) {
  return attn_sub_out_bytes(B, Hq, Hkv, P) +
         align256((size_t)B * P * attn_split(B, Hkv, P) * Hq * sizeof(float));
}

hipError_t launch_slice_merge(const float* so, const float* sl, int B, int P, int C, int Hq, float* part_out,
                              float* part_lse, float* out, float* out_lse, hipStream_t stream);

// The shares' partials go to the workspace; slice_merge_kernel then writes the slice
// partials and, when out != NULL, the merge of the slices.
hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* page_table,
                              const int32_t* lens, const int32_t* sel, const int32_t* sel_count, int B,
                              int Hq, int Hkv, int max_pages, int k, int P, float scale,
                              float* part_out, float* part_lse, float* out, float* out_lse,
                              void* workspace, int T, hipStream_t stream) {
  const int C = attn_split(B, Hkv, P);
  float* sub_out = static_cast<float*>(workspace);
  float* sub_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + attn_sub_out_bytes(B, Hq, Hkv, P));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(C * Hkv, P, B), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), page_table, lens, sel, sel_count, Hq, Hkv,
                     max_pages, k, P, C, T, scale_log2, sub_out, sub_lse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_slice_merge(sub_out, sub_lse, B, P, C, Hq, part_out, part_lse, out, out_lse, stream);
}

}  // namespace qsa
