// Fractal flatten and its inverse ("NABLA: Neighborhood Adaptive Block-Level
// Attention", gist.science, Methodology: token reordering).  Each P x P
// spatial patch of a frame becomes a contiguous run of 64 tokens; frames keep
// their order.  Pure data movement: one thread per 16-byte chunk of a token
// row, walking the blocked tensor in order so that its side is fully
// coalesced; the natural side is read or written in 8-token patch rows
// (1-2 KB contiguous).
#include "nabla_common.hpp"

namespace nabla {

namespace {

// grid.x covers the chunks of one head (< 2^31), grid.y strides over heads.
template <bool kInverse>
__global__ void __launch_bounds__(256) flatten_kernel(const Geo g, int cpt_log2,
                                                      const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst, int head_chunks,
                                                      int64_t thw_head_chunks) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // chunk inside the blocked head
  if (i >= head_chunks) return;
  const int c = i & ((1 << cpt_log2) - 1);
  const int tok = i >> cpt_log2;                          // slot in [nb, 64]
  const int s = tok & (kN - 1);
  const int b = tok >> 6;
  const BlockCoord bc = block_coord(g, b);
  const int hh = bc.hb * kP + (s >> 3);
  const int ww = bc.wb * kP + (s & 7);
  const bool valid = hh < g.H && ww < g.W;
  const int nat = (((bc.t * g.H + hh) * g.W + ww) << cpt_log2) + c;
  for (int64_t h = blockIdx.y; h < g.bh; h += gridDim.y) {
    const int64_t blk_off = h * head_chunks + i;
    const int64_t nat_off = h * thw_head_chunks + nat;
    if (!kInverse) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (valid) v = src[nat_off];
      dst[blk_off] = v;
    } else if (valid) {
      dst[nat_off] = src[blk_off];
    }
  }
}

}  // namespace

hipError_t launch_flatten(const Geo& g, int elem_bytes, const void* src, void* dst, bool inverse,
                          hipStream_t s) {
  const int cpt = g.d * elem_bytes / 16;                  // 8, 16 or 32 chunks per token
  const int cpt_log2 = cpt == 8 ? 3 : (cpt == 16 ? 4 : 5);
  const int head_chunks = g.nb * kN * cpt;
  const int64_t thw_head_chunks = (int64_t)g.T * g.H * g.W * cpt;
  const dim3 grid((head_chunks + 255) / 256, (unsigned)(g.bh < 65535 ? g.bh : 65535));
  if (!inverse) {
    hipLaunchKernelGGL(flatten_kernel<false>, grid, dim3(256), 0, s, g, cpt_log2,
                       (const u32x4*)src, (u32x4*)dst, head_chunks, thw_head_chunks);
  } else {
    hipLaunchKernelGGL(flatten_kernel<true>, grid, dim3(256), 0, s, g, cpt_log2,
                       (const u32x4*)src, (u32x4*)dst, head_chunks, thw_head_chunks);
  }
  return hipGetLastError();
}

}  // namespace nabla
