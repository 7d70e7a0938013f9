// Row-slab copies for the forward's kv-group mode: the q heads of one kv group
// (and that group's k/v head) are gathered from the packed [T, H, D] layout into
// contiguous slabs, and the slab's outputs are scattered back. Plain streaming
// copies, HBM-bound.
#include "moba_plan.h"

namespace moba {

// Copies `rows` rows of `per_row` units (16 or 4 bytes) from src (row stride
// sstride bytes) to dst (row stride dstride bytes). Workgroup b copies rows
// [b * rows_per_wg, ...), each thread every 256th unit of that range.
template <typename U>
__global__ void __launch_bounds__(256) k_copy_rows(const char* __restrict__ src, int64_t sstride,
                                                   char* __restrict__ dst, int64_t dstride,
                                                   int64_t rows, int per_row, int rows_per_wg) {
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
  if (r0 >= rows) return;
  const int nr = (int)min((int64_t)rows_per_wg, rows - r0);
  const int total = nr * per_row;
  for (int i = threadIdx.x; i < total; i += 256) {
    const int r = i / per_row, c = i - r * per_row;
    const U v = *reinterpret_cast<const U*>(src + (r0 + r) * sstride + (int64_t)sizeof(U) * c);
    *reinterpret_cast<U*>(dst + (r0 + r) * dstride + (int64_t)sizeof(U) * c) = v;
  }
}

hipError_t launch_copy_rows(const void* src, int64_t sstride, void* dst, int64_t dstride,
                            int64_t rows, int64_t width, hipStream_t s) {
  if (rows <= 0 || width <= 0) return hipSuccess;
  const bool wide = width % 16 == 0 && sstride % 16 == 0 && dstride % 16 == 0 &&
                    (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  const int unit = wide ? 16 : 4;
  const int per_row = (int)(width / unit);
  const int rows_per_wg = per_row >= 4096 ? 1 : 4096 / per_row;
  const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
  if (wide)
    hipLaunchKernelGGL(k_copy_rows<uint4>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const char*)src, sstride, (char*)dst, dstride, rows, per_row,
                       rows_per_wg);
  else
    hipLaunchKernelGGL(k_copy_rows<uint32_t>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const char*)src, sstride, (char*)dst, dstride, rows, per_row,
                       rows_per_wg);
  return hipGetLastError();
}

}  // namespace moba
