// check_pages.hip - device-side check of the page-table preconditions of every entry point.
//
// The compute kernels trust the page table and the lengths (checking them there would put a
// test on every gathered row). This kernel checks them once, reading only the table and the
// lengths, never a cache row, so a bad table cannot make it fault:
//   verdict[b] = -1  request b is valid: 0 <= L_b <= max_pages*page_size and every page id
//                    page_table[b][p] for p < ceil(L_b/page_size) lies in [0, num_pages)
//   verdict[b] = -2  L_b < 0 or L_b > max_pages*page_size (no page id is read)
//   verdict[b] = p   p >= 0 is the first page slot whose id is outside [0, num_pages)
// One workgroup of 256 threads per request; the first bad slot is the minimum over threads.
#include "qsa_device.h"

namespace qsa {

__global__ __launch_bounds__(256) void check_pages_kernel(const int32_t* __restrict__ page_table,
                                                          const int32_t* __restrict__ lens, int max_pages,
                                                          int page_size, int num_pages,
                                                          int32_t* __restrict__ verdict) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int L = lens[b];
  if (L < 0 || (long long)L > (long long)max_pages * page_size) {
    if (t == 0) verdict[b] = -2;
    return;
  }
  const int npages = (L + page_size - 1) / page_size;
  const int32_t* row = page_table + (size_t)b * max_pages;
  int first = 0x7FFFFFFF;
  for (int p = t; p < npages; p += 256) {
    const int id = row[p];
    if ((id < 0 || id >= num_pages) && p < first) first = p;
  }
  __shared__ int s_first;
  if (t == 0) s_first = 0x7FFFFFFF;
  __syncthreads();
  if (first != 0x7FFFFFFF) atomicMin(&s_first, first);
  __syncthreads();
  if (t == 0) verdict[b] = s_first == 0x7FFFFFFF ? -1 : s_first;
}

hipError_t launch_check_pages(const int32_t* page_table, const int32_t* lens, int B, int max_pages,
                              int page_size, int num_pages, int32_t* verdict, hipStream_t stream) {
  hipLaunchKernelGGL(check_pages_kernel, dim3(B), dim3(256), 0, stream, page_table, lens, max_pages,
                     page_size, num_pages, verdict);
  return hipGetLastError();
}

}  // namespace qsa
