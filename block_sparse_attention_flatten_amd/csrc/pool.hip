// Block average pooling of Q and K ("NABLA: Neighborhood Adaptive Block-Level
// Attention", gist.science, Methodology: downsampling; lsdiaocha.cn article,
// sec. 2 step 1): the delegate of a block is the mean of its valid tokens.
//
// HBM-bound streaming read, one wavefront per block (pool_block in
// mask_items.hpp; nabla_qkv_split repeats its summation order, so both give
// the same bits).  The pooled keys are written as the mask kernel reads
// them: each mean as three exact bf16 parts, in its tiled order.  Both the
// natural and the blocked layout are addressed in 8-token patch rows, so the
// reorder costs no extra pass.
#include "mask_items.hpp"

namespace nabla {

namespace {

using mask_detail::PoolShape;

template <typename T, int D>
__global__ void __launch_bounds__(256) pool_kernel(const Geo g, const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ qbar,
                                                   __bf16* __restrict__ kbar) {
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (head, block)
  if (gb >= g.bh * g.nb) return;
  const int64_t head = gb / g.nb;
  const int b = (int)(gb - head * g.nb);
  const T* x = (blockIdx.y == 0 ? q : k) + head * (int64_t)g.head_elems;
  float mean[PoolShape<T, D>::kElems];
  mask_detail::pool_block<T, D>(g, x, b, mean);
  if (blockIdx.y == 0)
    mask_detail::store_mean<T, D>(mean, qbar + gb * D);
  else
    mask_detail::store_mean_tiled<T, D>(mean, kbar + head * kbar_head_elems(g.nb, D), b);
}

template <typename T, int D>
hipError_t launch(const Geo& g, const void* q, const void* k, float* qbar, __bf16* kbar,
                  hipStream_t s) {
  const int64_t waves = g.bh * g.nb;
  const dim3 grid((unsigned)((waves + 3) / 4), 2);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, s, g, (const T*)q, (const T*)k,
                     qbar, kbar);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Geo& g, bool bf16, const void* q, const void* k, float* qbar,
                       __bf16* kbar, hipStream_t s) {
  if (bf16) {
    return g.d == 64 ? launch<__bf16, 64>(g, q, k, qbar, kbar, s)
                     : launch<__bf16, 128>(g, q, k, qbar, kbar, s);
  }
  return g.d == 64 ? launch<float, 64>(g, q, k, qbar, kbar, s)
                   : launch<float, 128>(g, q, k, qbar, kbar, s);
}

}  // namespace nabla
