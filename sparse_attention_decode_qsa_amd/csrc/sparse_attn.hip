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
// Work split. The kept blocks of a request are ascending, so those of slice p form one
// run of sel_blocks. A tile is 4 kept blocks (16 tokens) of one slice; a workgroup of 4
// waves ("split") takes 4 consecutive tiles of one slice for one KV head, one tile per
// wave. Grid: (splits, Hkv, B); each workgroup derives its slice and tiles from
// sel_blocks. A slice covered by one split writes its partial directly; otherwise each
// split stores (max, sum, unnormalised output) in the workspace and the last split of
// the slice to finish (atomic ticket, no waiting) merges them.
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

constexpr int kAttnWaves = 4;
constexpr int kTilesPerSplit = kAttnWaves;   // one 16-token tile per wave
constexpr int kRecFloats = 2 * kMaxGroup + kMaxGroup * kHeadDim;  // m[16], l[16], o[16][128]

__host__ __device__ inline int attn_max_splits(int k, int P) {
  // sum over slices of max(1, ceil(ntiles_p / T)) with sum ntiles_p <= ceil(k/4) + P
  return (k + 4 * kTilesPerSplit - 1) / (4 * kTilesPerSplit) + 2 * P;
}

__host__ __device__ inline size_t attn_ws_bytes(int B, int Hkv, int k, int P) {
  const size_t tickets = ((size_t)B * Hkv * P * 4 + 255) & ~(size_t)255;
  return tickets + (size_t)B * Hkv * attn_max_splits(k, P) * kRecFloats * 4;
}

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

__global__ __launch_bounds__(kAttnWaves * 64) void sparse_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int Hq, int Hkv,
    int max_pages, int k, int P, float scale_log2, float* __restrict__ part_out,
    float* __restrict__ part_lse, uint32_t* __restrict__ tickets, float* __restrict__ recs) {
  const int x = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = lane_id(), wave = t >> 6;
  const int group = Hq / Hkv;
  const int L = lens[b];
  const int K = sel_count[b];
  const int32_t* sb = sel + (size_t)b * k;

  __shared__ int s_seg[kMaxSlices + 1];
  __shared__ int s_pref[kMaxSlices + 1];
  __shared__ int s_flag;
  __shared__ float s_m[kAttnWaves][kMaxGroup];
  __shared__ float s_l[kAttnWaves][kMaxGroup];
  __shared__ float s_o[kAttnWaves][kMaxGroup][kHeadDim + 4];

  // Slice runs inside sel_blocks, and the splits of each slice.
  const int npages = (L + kPageSize - 1) / kPageSize;
  const int S = (npages + P - 1) / P;
  for (int p = t; p <= P; p += kAttnWaves * 64)
    s_seg[p] = lower_bound_i32(sb, K, min(p * S, npages) * kBlocksPerPage);
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int p = 0; p < P; ++p) {
      s_pref[p] = run;
      const int ntiles = (s_seg[p + 1] - s_seg[p] + 3) / 4;
      run += max(1, (ntiles + kTilesPerSplit - 1) / kTilesPerSplit);
    }
    s_pref[P] = run;
  }
  __syncthreads();
  if (x >= s_pref[P]) return;
  int p = 0;
  while (s_pref[p + 1] <= x) ++p;
  const int split = x - s_pref[p];
  const int nsplit = s_pref[p + 1] - s_pref[p];
  const int seg0 = s_seg[p], seg1 = s_seg[p + 1];

  const int i16 = lane & 15, q4 = lane >> 4;
  const int tile = split * kTilesPerSplit + wave;
  const int bbase = seg0 + 4 * tile;  // first kept-block slot of this tile

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

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (bbase < seg1) {
    // K operand: token i16 of the tile (block i16/4, row i16%4).
    bf16x8 ka[4];
    {
      const int slot = bbase + (i16 >> 2);
      const int tok = slot < seg1 ? 4 * sb[slot] + (i16 & 3) : L;
      if (tok < L) {
        const int page = page_table[(size_t)b * max_pages + (tok >> 6)];
        const uint16_t* krow = kc + (((size_t)page * kPageSize + (tok & 63)) * Hkv + g) * kHeadDim + 8 * q4;
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(krow + 32 * s);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) ka[s] = bf16x8{};
      }
    }
    // V operand: tokens of kept block q4 of the tile, dims 8*i16 .. +7.
    u16x8 vv[4];
    bool tv[4];
    {
      const int slot = bbase + q4;
      const int blk = slot < seg1 ? sb[slot] : -1;
      const int page = blk >= 0 ? page_table[(size_t)b * max_pages + (blk >> 4)] : 0;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tok = 4 * blk + v;
        tv[v] = blk >= 0 && tok < L;
        if (tv[v]) {
          const uint16_t* vrow = vc + (((size_t)page * kPageSize + (tok & 63)) * Hkv + g) * kHeadDim + 8 * i16;
          vv[v] = *reinterpret_cast<const u16x8*>(vrow);
        } else {
          vv[v] = u16x8{};
        }
      }
    }

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qa[s], sc, 0, 0, 0);

    float sv[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) sv[v] = tv[v] ? sc[v] * scale_log2 : -INFINITY;
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
      const uint32_t e0 = vv[0][u], e1 = vv[1][u], e2 = vv[2][u], e3 = vv[3][u];
      va.w[0] = pack2(e0, e1);
      va.w[1] = pack2(e2, e3);
      va.w[2] = va.w[0];
      va.w[3] = va.w[1];
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va.v, bp.v, acc[u], 0, 0, 0);
    }
  }

  // Wave partial -> LDS. Lane (q4, i16) holds head i16, dims 8*(4*q4 + r) + u.
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (q4 == 0) { s_m[wave][i16] = m_run; s_l[wave][i16] = l_tot; }
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_o[wave][i16][8 * (4 * q4 + r) + u] = acc[u][r];
  __syncthreads();

  // Combine the waves: thread -> (head, 8 dims).
  const int hh = t >> 4;            // 0..15
  const int d0 = (t & 15) * 8;      // 0..120
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][hh]);
  float Lsum = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
      const float mw = s_m[w][hh];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      Lsum += f * s_l[w][hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += f * s_o[w][hh][d0 + e];
    }
  }

  const int h_glob = g * group + hh;
  if (nsplit == 1) {
    if (hh < group) {
      float* dst = part_out + (((size_t)b * P + p) * Hq + h_glob) * kHeadDim + d0;
      const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = o[e] * inv;
      if (d0 == 0)
        part_lse[((size_t)b * P + p) * Hq + h_glob] =
            Lsum > 0.f ? (M + __log2f(Lsum)) * 0.69314718055994531f : -INFINITY;
    }
    return;
  }

  // Several splits: store this split's record, the last one of the slice merges.
  const int max_splits = gridDim.x;
  float* rec_base = recs + ((size_t)b * Hkv + g) * max_splits * kRecFloats;
  float* rec = rec_base + (size_t)x * kRecFloats;
  if (hh < group) {
#pragma unroll
    for (int e = 0; e < 8; ++e) rec[2 * kMaxGroup + hh * kHeadDim + d0 + e] = o[e];
    if (d0 == 0) { rec[hh] = M; rec[kMaxGroup + hh] = Lsum; }
  }
  __threadfence();
  __syncthreads();
  uint32_t* tk = tickets + ((size_t)b * Hkv + g) * P + p;
  if (t == 0) s_flag = atomicAdd(tk, 1u) == (uint32_t)(nsplit - 1);
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  if (hh < group) {
    const int x0 = s_pref[p];
    float MM = -INFINITY;
    for (int y = 0; y < nsplit; ++y)
      MM = fmaxf(MM, __hip_atomic_load(rec_base + (size_t)(x0 + y) * kRecFloats + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    float LL = 0.f, oo[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (MM != -INFINITY) {
      for (int y = 0; y < nsplit; ++y) {
        const float* ry = rec_base + (size_t)(x0 + y) * kRecFloats;
        const float my = __hip_atomic_load(ry + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (my == -INFINITY) continue;
        const float f = exp2f(my - MM);
        LL += f * __hip_atomic_load(ry + kMaxGroup + hh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          oo[e] += f * __hip_atomic_load(ry + 2 * kMaxGroup + hh * kHeadDim + d0 + e, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    float* dst = part_out + (((size_t)b * P + p) * Hq + h_glob) * kHeadDim + d0;
    const float inv = LL > 0.f ? 1.f / LL : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = oo[e] * inv;
    if (d0 == 0)
      part_lse[((size_t)b * P + p) * Hq + h_glob] =
          LL > 0.f ? (MM + __log2f(LL)) * 0.69314718055994531f : -INFINITY;
  }
  if (t == 0) *tk = 0;
}

size_t attn_workspace_bytes(int B, int Hkv, int k, int P) { return attn_ws_bytes(B, Hkv, k, P); }

hipError_t launch_sparse_attn(const void* q, const void* kc, const void* vc, const int32_t* page_table,
                              const int32_t* lens, const int32_t* sel, const int32_t* sel_count, int B,
                              int Hq, int Hkv, int max_pages, int k, int P, float scale,
                              float* part_out, float* part_lse, void* workspace, hipStream_t stream) {
  const int splits = attn_max_splits(k, P);
  char* ws = static_cast<char*>(workspace);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(ws);
  float* recs = reinterpret_cast<float*>(ws + (((size_t)B * Hkv * P * 4 + 255) & ~(size_t)255));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(sparse_attn_kernel, dim3(splits, Hkv, B), dim3(kAttnWaves * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), page_table, lens, sel, sel_count, Hq, Hkv,
                     max_pages, k, P, scale_log2, part_out, part_lse, tickets, recs);
  return hipGetLastError();
}

}  // namespace qsa
