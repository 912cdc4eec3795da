// calib_copy.hip - libqsa_calib: a plain device copy with the indexer scan's kind of loads
// (16-byte nontemporal loads, plain 16-byte stores), for calibrating byte counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qsa_calib.h"

namespace qsa_calib {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_copy_kernel(i32x4* __restrict__ dst, const i32x4* __restrict__ src,
                                                         size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = __builtin_nontemporal_load(src + i);
}

}  // namespace qsa_calib

extern "C" int qsa_calib_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return 0;
  if (!dst || !src) return 1;
  if ((bytes & 15u) != 0 || ((uintptr_t)dst & 15u) != 0 || ((uintptr_t)src & 15u) != 0) return 2;
  const size_t n16 = bytes / 16;
  size_t grid = (n16 + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(qsa_calib::calib_copy_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<qsa_calib::i32x4*>(dst), static_cast<const qsa_calib::i32x4*>(src), n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
