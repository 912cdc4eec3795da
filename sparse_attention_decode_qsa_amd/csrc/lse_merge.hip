// lse_merge.hip - K4: log-sum-exp merge of the P slice partials.
//
// Article "Qwen 4 QSA gets decode context parallelism: inside vLLM's draft PR for
// Qwen3.8-Flash-Next", section "What the pull request actually changes" (bullets) and
// section "Questions worth answering directly" (how DCP differs from TP): the partial
// attention results of the slices are combined after the split read. With M the largest
// finite slice lse and w_p = exp(lse_p - M):
//     out = sum_p w_p o_p / sum_p w_p,   lse = M + ln(sum_p w_p)
// Slices with lse = -inf carry no weight; with none finite, out = 0 and lse = -inf.
// One workgroup per (head, request), one thread per output dim.
#include "qsa_device.h"

namespace qsa {

__global__ __launch_bounds__(kHeadDim) void lse_merge_kernel(const float* __restrict__ po,
                                                             const float* __restrict__ pl, int P,
                                                             int Hq, float* __restrict__ out,
                                                             float* __restrict__ out_lse) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const float* lse = pl + (size_t)b * P * Hq + h;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, lse[(size_t)p * Hq]);
  float wsum = 0.f, acc = 0.f;
  if (M != -INFINITY) {
    for (int p = 0; p < P; ++p) {
      const float l = lse[(size_t)p * Hq];
      if (l == -INFINITY) continue;
      const float w = __expf(l - M);
      wsum += w;
      acc += w * po[(((size_t)b * P + p) * Hq + h) * kHeadDim + d];
    }
  }
  out[((size_t)b * Hq + h) * kHeadDim + d] = wsum > 0.f ? acc / wsum : 0.f;
  if (out_lse && d == 0) out_lse[(size_t)b * Hq + h] = wsum > 0.f ? M + __logf(wsum) : -INFINITY;
}

hipError_t launch_lse_merge(const float* po, const float* pl, int B, int P, int Hq, float* out,
                            float* out_lse, hipStream_t stream) {
  hipLaunchKernelGGL(lse_merge_kernel, dim3(Hq, B), dim3(kHeadDim), 0, stream, po, pl, P, Hq, out,
                     out_lse);
  return hipGetLastError();
}

}  // namespace qsa
