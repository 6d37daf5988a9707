// Layout pass after a transformer layer's fused QKV projection, with the
// NABLA block means computed on the way ("NABLA: Neighborhood Adaptive
// Block-Level Attention", gist.science, Methodology: token reordering and
// downsampling).  When the token sequence stays in the blocked (fractal-
// flattened) order across the network, the projection output is token-major
// [B, nb * 64, 3, heads, d]; the attention calls take head-major tensors.
// This pass reads each (block, head) tile once and writes
//   q, k   head-major copies in the blocked layout,
//   V^T    the attention kernel's transposed V operand (as nabla_transpose_v),
//   q̄, k̄   the means of the block's valid tokens (as nabla_pool, same bits
//          and the same split, tiled encoding for k̄),
// so pooling and the V transpose cost no pass of their own.
//
// One workgroup per (block, head, batch): the 3 x 64 token rows are read with
// 16-byte loads (each token's row of one head is contiguous), q and k chunks
// are written straight back out, and all three tiles are staged in LDS with
// pad slots zeroed.  Wavefronts 0 and 1 then form the q and k means in
// exactly the order of the pooling kernel (the same lane-to-chunk map,
// patch rows ascending, the same butterfly), and all four write V^T.
#include "mask_items.hpp"

namespace nabla {

namespace {

using mask_detail::PoolShape;

template <int D>
__global__ void __launch_bounds__(256) qkv_split_kernel(const Geo g, int heads,
                                                        const __bf16* __restrict__ qkv,
                                                        __bf16* __restrict__ q,
                                                        __bf16* __restrict__ k,
                                                        __bf16* __restrict__ vt,
                                                        float* __restrict__ qbar,
                                                        __bf16* __restrict__ kbar) {
  using S = PoolShape<__bf16, D>;
  constexpr int kChunks = D / 8;                 // 16-byte chunks per token row
  constexpr int kStride = D + 8;                 // LDS row stride (elements)
  __shared__ __attribute__((aligned(16))) __bf16 tile[3][kN * kStride];
  const int b = blockIdx.x;
  const int64_t head = (int64_t)blockIdx.z * heads + blockIdx.y;
  const BlockCoord bc = block_coord(g, b);
  const int rv = block_rows_valid(g, bc), cv = block_cols_valid(g, bc);
  const int64_t tok_elems = (int64_t)3 * heads * D;          // one token's q, k, v rows
  const __bf16* src =
      qkv + ((int64_t)blockIdx.z * g.nb + b) * kN * tok_elems + (int64_t)blockIdx.y * D;
  const int64_t out_base = head * (int64_t)g.head_elems + (int64_t)b * kN * D;

  for (int c = threadIdx.x; c < 3 * kN * kChunks; c += 256) {
    const int m = c / (kN * kChunks);            // 0: q, 1: k, 2: v
    const int rem = c - m * (kN * kChunks);
    const int t = rem / kChunks, ch = rem - t * kChunks;
    u32x4 x = *(const u32x4*)(src + t * tok_elems + (int64_t)m * heads * D + ch * 8);
    if (m == 0) *(u32x4*)(q + out_base + t * D + ch * 8) = x;
    if (m == 1) *(u32x4*)(k + out_base + t * D + ch * 8) = x;
    if (!((t >> 3) < rv && (t & 7) < cv)) x = u32x4{0u, 0u, 0u, 0u};   // pad slot
    *(u32x4*)(&tile[m][t * kStride + ch * 8]) = x;
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave < 2) {
    // lane: chunk of the row, first patch column; slot order as the pooling
    // kernel's loads: patch rows ascending, then the lane's patch columns
    constexpr int P = kP / S::kRowsPerLoad;
    const int chunk = lane % S::kLanesPerRow;
    const int row0 = lane / S::kLanesPerRow;
    float mean[S::kElems];
#pragma unroll
    for (int e = 0; e < S::kElems; ++e) mean[e] = 0.f;
#pragma unroll
    for (int i = 0; i < kP; ++i)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int t = kP * i + row0 + S::kRowsPerLoad * p;
        const u32x4 raw = *(const u32x4*)(&tile[wave][t * kStride + chunk * 8]);
        mask_detail::pool_accumulate<__bf16>(mean, raw);
      }
#pragma unroll
    for (int off = S::kLanesPerRow; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < S::kElems; ++e) mean[e] += __shfl_xor(mean[e], off);
    }
    const float inv = 1.0f / (float)(rv * cv);
#pragma unroll
    for (int e = 0; e < S::kElems; ++e) mean[e] *= inv;
    if (wave == 0)
      mask_detail::store_mean<__bf16, D>(mean, qbar + (head * g.nb + b) * D);
    else
      mask_detail::store_mean_tiled<__bf16, D>(mean, kbar + head * kbar_head_elems(g.nb, D), b);
  }

  // V^T: row = channel, keys permuted inside each group of 16 by swapping
  // bits 2 and 3 of the position (the attention kernel's operand order)
  __bf16* dst = vt + (head * g.nb + b) * (int64_t)(kN * D);
  for (int c = threadIdx.x; c < D * 8; c += 256) {
    const int ch = c >> 3, j = c & 7;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = 8 * j + e;
      const int key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1);
      out[e] = tile[2][key * kStride + ch];
    }
    *(bf16x8*)(dst + ch * kN + 8 * j) = out;
  }
}

}  // namespace

hipError_t launch_qkv_split(const Geo& g, int batch, int heads, const void* qkv, void* q, void* k,
                            void* vt, float* qbar, __bf16* kbar, hipStream_t s) {
  const dim3 grid((unsigned)g.nb, (unsigned)heads, (unsigned)batch);
  if (g.d == 64) {
    hipLaunchKernelGGL(qkv_split_kernel<64>, grid, dim3(256), 0, s, g, heads,
                       (const __bf16*)qkv, (__bf16*)q, (__bf16*)k, (__bf16*)vt, qbar, kbar);
  } else {
    hipLaunchKernelGGL(qkv_split_kernel<128>, grid, dim3(256), 0, s, g, heads,
                       (const __bf16*)qkv, (__bf16*)q, (__bf16*)k, (__bf16*)vt, qbar, kbar);
  }
  return hipGetLastError();
}

}  // namespace nabla
