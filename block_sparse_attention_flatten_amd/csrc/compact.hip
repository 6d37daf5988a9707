// Compressed kept-block lists (lsdiaocha.cn article on NABLA, sec. 5: only the
// compressed sparse matrix is stored instead of the full S x S map).
//
// Per head: row_ptr = exclusive prefix sum of the row counts, col_idx = kept
// block indices of each row in ascending order.  Each wavefront compacts
// kCompactRows rows of one head (compact_rows in mask_items.hpp).
#include "mask_items.hpp"

namespace nabla {

namespace {

constexpr int kWaves = 4;

__global__ void __launch_bounds__(kWaves * 64) compact_kernel(const Geo g,
                                                              const mask_detail::CompactArgs a,
                                                              int units_per_head) {
  const int64_t unit = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (unit >= g.bh * units_per_head) return;
  const int64_t head = unit / units_per_head;
  const int r0 = (int)(unit - head * units_per_head) * mask_detail::kCompactRows;
  mask_detail::compact_rows(g, a, head, r0, mask_detail::kCompactRows);
}

}  // namespace

hipError_t launch_compact(const Geo& g, const uint32_t* bits, const int32_t* cnt,
                          int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  const mask_detail::CompactArgs a = {bits, cnt, row_ptr, col_idx};
  const int per_head = (g.nb + mask_detail::kCompactRows - 1) / mask_detail::kCompactRows;
  const int64_t units = g.bh * per_head;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)((units + kWaves - 1) / kWaves)),
                     dim3(kWaves * 64), 0, s, g, a, per_head);
  return hipGetLastError();
}

}  // namespace nabla
