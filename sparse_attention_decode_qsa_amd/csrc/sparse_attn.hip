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
// Work split. One workgroup of 16 waves per (request, slice, KV head); nothing is shared
// between workgroups. The kept blocks are ascending, so those of slice p form one run of
// sel_blocks, found by two binary searches in LDS. A tile is 4 kept blocks (16 tokens); tiles
// are dealt round-robin to the waves and each wave keeps an online softmax over its
// tiles. The 16 wave partials are merged in LDS by a 4-round tree (deterministic order).
// The request's kept ids and the page of each kept block of the slice are staged in LDS
// first, so a tile needs no dependent global loads besides its K/V rows.
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
// Masked tokens (past the slice's run or past L_b) are never loaded: their K and V
// registers stay zero and their scores are -inf, so NaN rows cannot leak in.
#include "qsa_device.h"

namespace qsa {

constexpr int kAttnWaves = 16;

__device__ __forceinline__ int lower_bound_i32(const int32_t* a, int n, int v) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < v) lo = mid + 1; else hi = mid;
  }
  return lo;
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

// Tile of 4 kept blocks starting at slot bbase of the slice's run [seg0, seg1); block ids
// and their page ids come from LDS.
__device__ __forceinline__ void load_tile(Tile& T, int bbase, int seg0, int seg1, const int* s_sel,
                                          const int* s_page, int L, const uint16_t* kc,
                                          const uint16_t* vc, int Hkv, int g, int i16, int q4) {
  {
    const int slot = bbase + (i16 >> 2);
    const int tok = slot < seg1 ? 4 * s_sel[slot] + (i16 & 3) : L;
    if (tok < L) {
      const int page = s_page[slot - seg0];
      const uint16_t* krow = kc + (((size_t)page * kPageSize + (tok & 63)) * Hkv + g) * kHeadDim + 8 * q4;
#pragma unroll
      for (int s = 0; s < 4; ++s) T.k[s] = *reinterpret_cast<const bf16x8*>(krow + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) T.k[s] = bf16x8{};
    }
  }
  const int slot = bbase + q4;
  const int blk = slot < seg1 ? s_sel[slot] : -1;
  const int page = blk >= 0 ? s_page[slot - seg0] : 0;
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

__global__ __launch_bounds__(kAttnWaves * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int Hq, int Hkv,
    int max_pages, int k, int P, float scale_log2, float* __restrict__ part_out,
    float* __restrict__ part_lse) {
  const int g = blockIdx.x, p = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int i16 = lane & 15, q4 = lane >> 4;
  const int group = Hq / Hkv;
  const int L = lens[b];
  const int K = sel_count[b];
  const int32_t* sb = sel + (size_t)b * k;
  const int32_t* ptab = page_table + (size_t)b * max_pages;

  __shared__ int s_seg[2];
  __shared__ int s_sel[kMaxK];      // kept block ids of the request
  __shared__ int s_page[kMaxK];     // physical page of each kept block of this slice
  __shared__ float s_m[kAttnWaves / 2][kMaxGroup];
  __shared__ float s_l[kAttnWaves / 2][kMaxGroup];
  __shared__ float s_o[kAttnWaves / 2][kMaxGroup][kHeadDim + 4];

  // The request's kept ids and this thread's Q operand are loaded in one round.
  for (int i = t; i < K; i += kAttnWaves * 64) s_sel[i] = sb[i];
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

  // Run of kept blocks inside this slice, then the page of each of them.
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int S = (npages + P - 1) / P;
  if (t < 2) s_seg[t] = lower_bound_i32(s_sel, K, min((p + t) * S, npages) * kBlocksPerPage);
  __syncthreads();
  const int seg0 = s_seg[0], seg1 = s_seg[1];
  const int ntiles = (seg1 - seg0 + 3) / 4;
  for (int i = seg0 + t; i < seg1; i += kAttnWaves * 64) s_page[i - seg0] = ptab[s_sel[i] >> 4];
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int tile = wave; tile < ntiles; tile += kAttnWaves) {
    Tile cur;
    load_tile(cur, seg0 + 4 * tile, seg0, seg1, s_sel, s_page, L, kc, vc, Hkv, g, i16, q4);

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[s], qa[s], sc, 0, 0, 0);

    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = cur.tv[v] ? sc[v] * scale_log2 : -INFINITY;
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
      va.w[0] = pack2(cur.v[0][u], cur.v[1][u]);
      va.w[1] = pack2(cur.v[2][u], cur.v[3][u]);
      va.w[2] = va.w[0];
      va.w[3] = va.w[1];
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, bp.v, acc[u], 0, 0, 0);
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);

  // Tree merge of the wave partials: in round r the upper half of the live waves hands
  // (m, l, O) to the lower half through LDS. Lane (q4, i16) holds head i16 and dims
  // 8*(4*q4 + r) + u in acc[u][r].
  for (int half = kAttnWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      const int w = wave - half;
      if (q4 == 0) { s_m[w][i16] = m_run; s_l[w][i16] = l_tot; }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_o[w][i16][8 * (4 * q4 + r) + u] = acc[u][r];
    }
    __syncthreads();
    if (wave < half) {
      const float mo = s_m[wave][i16], lo = s_l[wave][i16];
      const float M = fmaxf(m_run, mo);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float fa = exp2f(m_run - Mu), fb = exp2f(mo - Mu);
      l_tot = l_tot * fa + lo * fb;
      m_run = M;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[u][r] = acc[u][r] * fa + s_o[wave][i16][8 * (4 * q4 + r) + u] * fb;
    }
    __syncthreads();
  }

  if (wave == 0 && i16 < group) {
    const int h = g * group + i16;
    float* dst = part_out + (((size_t)b * P + p) * Hq + h) * kHeadDim + 32 * q4;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      f32x4 lo4, hi4;
#pragma unroll
      for (int u = 0; u < 4; ++u) { lo4[u] = acc[u][r] * inv; hi4[u] = acc[u + 4][r] * inv; }
      *reinterpret_cast<f32x4*>(dst + 8 * r) = lo4;
      *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = hi4;
    }
    if (q4 == 0)
      part_lse[((size_t)b * P + p) * Hq + h] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
  }
}

size_t attn_workspace_bytes(int B, int Hkv, int k, int P) {
  (void)B;
  (void)Hkv;
  (void)k;
  (void)P;
  return 0;
}

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* page_table,
                              const int32_t* lens, const int32_t* sel, const int32_t* sel_count, int B,
                              int Hq, int Hkv, int max_pages, int k, int P, float scale,
                              float* part_out, float* part_lse, void* workspace, hipStream_t stream) {
  (void)workspace;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(Hkv, P, B), dim3(kAttnWaves * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), page_table, lens, sel, sel_count, Hq, Hkv,
                     max_pages, k, P, scale_log2, part_out, part_lse);
  return hipGetLastError();
}

}  // namespace qsa
