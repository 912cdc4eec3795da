// lse_merge.hip - K4: log-sum-exp merge of partial attention results.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes" (bullets) and
// section "Questions worth answering directly" (how DCP differs from TP): the per-slice
// partials are joined once every slice has been read. With M the largest
// finite slice lse and w_p = exp(lse_p - M):
//     out = sum_p w_p o_p / sum_p w_p,   lse = M + ln(sum_p w_p)
// Slices with lse = -inf carry no weight; with none finite, out = 0 and lse = -inf.
//
// lse_merge_kernel merges given slice partials. slice_merge_kernel first forms every slice
// partial from the partials of its C shares (the same formula over the shares), writes it,
// and then merges the slices exactly as lse_merge_kernel does (same operations in the same
// order), so the fused chain and the separate calls give the same bits.
// One workgroup per (head, request), one thread per output dim.
#include "qsa_device.h"

namespace qsa {

constexpr int kMaxShares = 32;  // shares per slice (at most the attention kernel's split)

__global__ __launch_bounds__(kHeadDim) void lse_merge_kernel(const float* __restrict__ po,
                                                             const float* __restrict__ pl, int P,
                                                             int Hq, float* __restrict__ out,
                                                             float* __restrict__ out_lse) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* lse = pl + (size_t)b * P * Hq + h;
  // The first 64 slice lse values come in by one vector load per wave (lane p holds slice p)
  // and are read out as wave-uniform values; slices past 64 are read directly.
  const int lane = threadIdx.x & 63;
  const int lse_lane = __float_as_int(lane < P ? lse[(size_t)lane * Hq] : -INFINITY);
  auto lse_of = [&](int p) {
    return p < 64 ? __int_as_float(__builtin_amdgcn_readlane(lse_lane, p)) : lse[(size_t)p * Hq];
  };
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, lse_of(p));
  float wsum = 0.f, acc = 0.f;
  if (M != -INFINITY) {
#pragma unroll 8
    for (int p = 0; p < P; ++p) {
      const float v = po[(((size_t)b * P + p) * Hq + h) * kHeadDim + d];   // loaded in batches
      const float l = lse_of(p);
      if (l == -INFINITY) continue;
      const float w = __expf(l - M);
      wsum += w;
      acc += w * v;
    }
  }
  out[((size_t)b * Hq + h) * kHeadDim + d] = wsum > 0.f ? acc / wsum : 0.f;
  if (out_lse && d == 0) out_lse[(size_t)b * Hq + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

// so [B, P, C, Hq, 128], sl [B, P, C, Hq] -> part_out [B, P, Hq, 128], part_lse [B, P, Hq]
// (not written when part_out is NULL: with C = 1 the attention kernel wrote them as so, sl);
// then, when out != NULL, out [B, Hq, 128] and (when out_lse != NULL) out_lse [B, Hq].
// Slice p: Mp = max_c lse_pc, w_c = exp(lse_pc - Mp) over the finite shares,
//   part_out = sum_c w_c o_pc / sum_c w_c,  part_lse = Mp + ln(sum_c w_c)   (0, -inf if none)
// then the slices are merged with the operations of lse_merge_kernel, in the same order.
constexpr int kFastShares = 32;

// P * C <= kFastShares: each thread loads every share value of its dim at entry (the share
// lse values arrive by one vector load per wave), and combines them in registers.
template <int C>
__device__ __forceinline__ void slice_merge_regs(const float* __restrict__ so, const float* __restrict__ sl,
                                                 int P, int Hq, int h, int b, int d, float* __restrict__ part_out,
                                                 float* __restrict__ part_lse, float* __restrict__ out,
                                                 float* __restrict__ out_lse) {
  constexpr int PM = kFastShares / C;
  const int n = P * C;
  const float* col = so + ((size_t)b * n * Hq + h) * kHeadDim + d;   // share i at col[i * Hq * 128]
  const float* lcol = sl + (size_t)b * n * Hq + h;                   // share i at lcol[i * Hq]
  const size_t stride = (size_t)Hq * kHeadDim;
  // One vector load brings the n <= 32 share lse values into lanes 0..n-1 (then read out as
  // wave-uniform values); the share values are loaded without branches (a share past n reads
  // share 0 and is never used: its lse is -inf).
  const int lane = threadIdx.x & 63;
  const float lse_lane = lane < n ? lcol[(size_t)lane * Hq] : -INFINITY;
  float lv[kFastShares], v[kFastShares];
#pragma unroll
  for (int i = 0; i < kFastShares; ++i) v[i] = col[(i < n ? i : 0) * stride];
#pragma unroll
  for (int i = 0; i < kFastShares; ++i)
    lv[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lse_lane), i));
  float mp[PM], lp[PM];
#pragma unroll
  for (int p = 0; p < PM; ++p) {
    float Mp = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) Mp = fmaxf(Mp, lv[p * C + c]);
    float ws = 0.f;
    if (Mp != -INFINITY) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (lv[p * C + c] != -INFINITY) ws += __expf(lv[p * C + c] - Mp);
    }
    mp[p] = Mp;
    lp[p] = ws > 0.f ? Mp + __logf(ws) : -INFINITY;
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < PM; ++p) M = fmaxf(M, lp[p]);   // slices past P hold -inf
  float wsum = 0.f, acc = 0.f;
#pragma unroll
  for (int p = 0; p < PM; ++p) {
    if (p >= P) break;
    float ws = 0.f, a = 0.f;
    if (mp[p] != -INFINITY) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float l = lv[p * C + c];
        if (l == -INFINITY) continue;
        const float w = __expf(l - mp[p]);
        ws += w;
        a += w * v[p * C + c];
      }
    }
    const float o = ws > 0.f ? a / ws : 0.f;
    if (part_out) {
      part_out[(((size_t)b * P + p) * Hq + h) * kHeadDim + d] = o;
      if (d == 0) part_lse[((size_t)b * P + p) * Hq + h] = lp[p];
    }
    if (M != -INFINITY && lp[p] != -INFINITY) {
      const float w = __expf(lp[p] - M);
      wsum += w;
      acc += w * o;
    }
  }
  if (out) {
    out[((size_t)b * Hq + h) * kHeadDim + d] = wsum > 0.f ? acc / wsum : 0.f;
    if (out_lse && d == 0) out_lse[(size_t)b * Hq + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
  }
}

// P * C <= 8 (every slice in one share, as with many virtual requests): the same operations,
// four dims per thread (16-byte loads and stores), four heads per workgroup of 128 threads.
template <int C>
__global__ __launch_bounds__(128) void slice_merge_v4_kernel(const float* __restrict__ so,
                                                             const float* __restrict__ sl, int P, int Hq,
                                                             float* __restrict__ part_out,
                                                             float* __restrict__ part_lse,
                                                             float* __restrict__ out,
                                                             float* __restrict__ out_lse) {
  constexpr int NV = 8;
  constexpr int PM = NV / C;
  const int h = blockIdx.x * 4 + (threadIdx.x >> 5), b = blockIdx.y, d0 = 4 * (threadIdx.x & 31);
  if (h >= Hq) return;
  const int n = P * C;
  const float* col = so + ((size_t)b * n * Hq + h) * kHeadDim + d0;
  const float* lcol = sl + (size_t)b * n * Hq + h;
  const size_t stride = (size_t)Hq * kHeadDim;
  // The n <= NV share lse values: a wave holds two heads (lanes 0-31 and 32-63), and lane
  // 32*half + i loads share i of its half's head, so one vector load brings both heads' values;
  // each half reads its own lanes (two uniform reads, one select). The share values are loaded
  // without branches (a share past n reads share 0 and is never used).
  const int sub = threadIdx.x & 31;
  const bool upper = (threadIdx.x & 32) != 0;
  const int lse_lane = __float_as_int(sub < n ? lcol[(size_t)sub * Hq] : -INFINITY);
  float lv[NV];
  f32x4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = *reinterpret_cast<const f32x4*>(col + (i < n ? i : 0) * stride);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int lo = __builtin_amdgcn_readlane(lse_lane, i), hi = __builtin_amdgcn_readlane(lse_lane, 32 + i);
    lv[i] = __int_as_float(upper ? hi : lo);
  }
  float mp[PM], lp[PM];
#pragma unroll
  for (int p = 0; p < PM; ++p) {
    float Mp = -INFINITY;
#pragma unroll
    for (int c = 0; c < C; ++c) Mp = fmaxf(Mp, lv[p * C + c]);
    float ws = 0.f;
    if (Mp != -INFINITY) {
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (lv[p * C + c] != -INFINITY) ws += __expf(lv[p * C + c] - Mp);
    }
    mp[p] = Mp;
    lp[p] = ws > 0.f ? Mp + __logf(ws) : -INFINITY;
  }
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < PM; ++p) M = fmaxf(M, lp[p]);
  float wsum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < PM; ++p) {
    if (p >= P) break;
    float ws = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (mp[p] != -INFINITY) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float l = lv[p * C + c];
        if (l == -INFINITY) continue;
        const float w = __expf(l - mp[p]);
        ws += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] += w * v[p * C + c][e];
      }
    }
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = ws > 0.f ? a[e] / ws : 0.f;
    if (part_out) {
      *reinterpret_cast<f32x4*>(part_out + (((size_t)b * P + p) * Hq + h) * kHeadDim + d0) = o;
      if (d0 == 0) part_lse[((size_t)b * P + p) * Hq + h] = lp[p];
    }
    if (M != -INFINITY && lp[p] != -INFINITY) {
      const float w = __expf(lp[p] - M);
      wsum += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += w * o[e];
    }
  }
  if (out) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = wsum > 0.f ? acc[e] / wsum : 0.f;
    *reinterpret_cast<f32x4*>(out + ((size_t)b * Hq + h) * kHeadDim + d0) = r;
    if (out_lse && d0 == 0) out_lse[(size_t)b * Hq + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
  }
}

// Any P * C: the share lse values go through LDS, and slice p+1's share values are loaded
// while slice p is combined.
template <int C>
__device__ __forceinline__ void slice_merge_lds(const float* __restrict__ so, const float* __restrict__ sl,
                                                int P, int Hq, int h, int b, int d,
                                                float* __restrict__ part_out, float* __restrict__ part_lse,
                                                float* __restrict__ out, float* __restrict__ out_lse) {
  const int n = P * C;
  const float* col = so + ((size_t)b * n * Hq + h) * kHeadDim + d;
  const size_t stride = (size_t)Hq * kHeadDim;
  __shared__ float s_share_lse[kMaxSlices * kMaxShares];
  __shared__ float s_slice_max[kMaxSlices];
  __shared__ float s_slice_lse[kMaxSlices];
  for (int i = d; i < n; i += kHeadDim) s_share_lse[i] = sl[((size_t)b * n + i) * Hq + h];
  __syncthreads();
  if (d < P) {
    float Mp = -INFINITY;
    for (int c = 0; c < C; ++c) Mp = fmaxf(Mp, s_share_lse[d * C + c]);
    float ws = 0.f;
    if (Mp != -INFINITY)
      for (int c = 0; c < C; ++c) {
        const float l = s_share_lse[d * C + c];
        if (l != -INFINITY) ws += __expf(l - Mp);
      }
    s_slice_max[d] = Mp;
    s_slice_lse[d] = ws > 0.f ? Mp + __logf(ws) : -INFINITY;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, s_slice_lse[p]);
  float cur[C], nxt[C];
#pragma unroll
  for (int c = 0; c < C; ++c) cur[c] = col[c * stride];
  float wsum = 0.f, acc = 0.f;
  for (int p = 0; p < P; ++p) {
    if (p + 1 < P) {
#pragma unroll
      for (int c = 0; c < C; ++c) nxt[c] = col[((size_t)(p + 1) * C + c) * stride];
    }
    const float Mp = s_slice_max[p];
    float ws = 0.f, a = 0.f;
    if (Mp != -INFINITY) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float l = s_share_lse[p * C + c];
        if (l == -INFINITY) continue;
        const float w = __expf(l - Mp);
        ws += w;
        a += w * cur[c];
      }
    }
    const float o = ws > 0.f ? a / ws : 0.f;
    const float lp = s_slice_lse[p];
    if (part_out) {
      part_out[(((size_t)b * P + p) * Hq + h) * kHeadDim + d] = o;
      if (d == 0) part_lse[((size_t)b * P + p) * Hq + h] = lp;
    }
    if (M != -INFINITY && lp != -INFINITY) {
      const float w = __expf(lp - M);
      wsum += w;
      acc += w * o;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) cur[c] = nxt[c];
  }
  if (out) {
    out[((size_t)b * Hq + h) * kHeadDim + d] = wsum > 0.f ? acc / wsum : 0.f;
    if (out_lse && d == 0) out_lse[(size_t)b * Hq + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
  }
}

// C is 1, 2, 4, 8, 16 or 32.
__global__ __launch_bounds__(kHeadDim) void slice_merge_kernel(const float* __restrict__ so,
                                                               const float* __restrict__ sl, int P, int C,
                                                               int Hq, float* __restrict__ part_out,
                                                               float* __restrict__ part_lse,
                                                               float* __restrict__ out,
                                                               float* __restrict__ out_lse) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
#define QSA_MERGE_C(CC)                                                                         \
  if (P * C <= kFastShares) slice_merge_regs<CC>(so, sl, P, Hq, h, b, d, part_out, part_lse, out, out_lse); \
  else slice_merge_lds<CC>(so, sl, P, Hq, h, b, d, part_out, part_lse, out, out_lse);                      \
  return
  switch (C) {
    case 1: QSA_MERGE_C(1);
    case 2: QSA_MERGE_C(2);
    case 4: QSA_MERGE_C(4);
    case 8: QSA_MERGE_C(8);
    case 16: QSA_MERGE_C(16);
    default: QSA_MERGE_C(32);
  }
#undef QSA_MERGE_C
}

hipError_t launch_lse_merge(const float* po, const float* pl, int B, int P, int Hq, float* out,
                            float* out_lse, hipStream_t stream) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(Hq, B), dim3(kHeadDim), 0, stream, po, pl, P, Hq, out,
                     out_lse);
  return hipGetLastError();
}

hipError_t launch_slice_merge(const float* so, const float* sl, int B, int P, int C, int Hq, float* part_out,
                              float* part_lse, float* out, float* out_lse, hipStream_t stream) {
  if ((C != 1 && C != 2 && C != 4 && C != 8 && C != 16 && C != 32) || P > kMaxSlices) return hipErrorInvalidValue;
  if (P * C <= 8) {
    const dim3 grid((Hq + 3) / 4, B);
    switch (C) {
      case 1: hipLaunchKernelGGL(slice_merge_v4_kernel<1>, grid, dim3(128), 0, stream, so, sl, P, Hq, part_out,
                                 part_lse, out, out_lse); break;
      case 2: hipLaunchKernelGGL(slice_merge_v4_kernel<2>, grid, dim3(128), 0, stream, so, sl, P, Hq, part_out,
                                 part_lse, out, out_lse); break;
      case 4: hipLaunchKernelGGL(slice_merge_v4_kernel<4>, grid, dim3(128), 0, stream, so, sl, P, Hq, part_out,
                                 part_lse, out, out_lse); break;
      default: hipLaunchKernelGGL(slice_merge_v4_kernel<8>, grid, dim3(128), 0, stream, so, sl, P, Hq, part_out,
                                  part_lse, out, out_lse); break;
    }
  } else {
    hipLaunchKernelGGL(slice_merge_kernel, dim3(Hq, B), dim3(kHeadDim), 0, stream, so, sl, P, C, Hq, part_out,
                       part_lse, out, out_lse);
  }
  return hipGetLastError();
}

}  // namespace qsa
