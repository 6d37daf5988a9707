// V in the blocked, transposed layout the attention kernel reads as matrix
// core operands: [B, heads, nb, d, 64] -- for every block, row c holds
// channel c of the block's 64 key tokens, keys permuted inside each group of
// 16 by swapping bits 2 and 3 of the position (positions 0-3, 4-7, 8-11,
// 12-15 hold keys 0-3, 8-11, 4-7, 12-15).  With that order one 16-byte row
// read gives a lane the 8 keys its v_mfma_f32_32x32x16_bf16 operand needs.
// Pad key slots are written as zeros.
//
// One workgroup per (head, block): the 64 x d tile is read with 16-byte
// loads (coalesced patch rows), staged in LDS, and written out as d rows of
// 64 keys, 16 bytes per thread.
#include "nabla_common.hpp"

namespace nabla {

namespace {

template <int D>
__global__ void __launch_bounds__(256) transpose_v_kernel(const Geo g,
                                                          const __bf16* __restrict__ v,
                                                          __bf16* __restrict__ vt) {
  constexpr int kStride = D + 8;                 // LDS row stride (elements)
  constexpr int kChunks = D / 8;                 // 16-byte chunks per token row
  __shared__ __attribute__((aligned(16))) __bf16 tile[kN * kStride];
  const int b = blockIdx.x;
  const int64_t head = blockIdx.y;
  const BlockCoord bc = block_coord(g, b);
  const int rv = block_rows_valid(g, bc), cv = block_cols_valid(g, bc);
  const __bf16* src = v + head * (int64_t)g.head_elems + block_base(g, b, bc);
  const int row_step = block_row_step(g);
  for (int c = threadIdx.x; c < kN * kChunks; c += 256) {
    const int r = c / kChunks, ch = c % kChunks;
    u32x4 x = {0u, 0u, 0u, 0u};
    if ((r >> 3) < rv && (r & 7) < cv) x = *(const u32x4*)(src + (r >> 3) * row_step + (r & 7) * D + ch * 8);
    *(u32x4*)(tile + r * kStride + ch * 8) = x;
  }
  __syncthreads();
  __bf16* dst = vt + (head * g.nb + b) * (int64_t)(kN * D);
  for (int c = threadIdx.x; c < D * 8; c += 256) {   // output row = channel, 8 chunks of 8 keys
    const int ch = c >> 3, j = c & 7;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = 8 * j + e;
      const int key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1);   // swap bits 2, 3
      out[e] = tile[key * kStride + ch];
    }
    *(bf16x8*)(dst + ch * kN + 8 * j) = out;
  }
}

}  // namespace

hipError_t launch_transpose_v(const Geo& g, const void* v, void* vt, hipStream_t s) {
  const dim3 grid((unsigned)g.nb, (unsigned)g.bh);
  if (g.d == 64) {
    hipLaunchKernelGGL(transpose_v_kernel<64>, grid, dim3(256), 0, s, g, (const __bf16*)v,
                       (__bf16*)vt);
  } else {
    hipLaunchKernelGGL(transpose_v_kernel<128>, grid, dim3(256), 0, s, g, (const __bf16*)v,
                       (__bf16*)vt);
  }
  return hipGetLastError();
}

}  // namespace nabla
