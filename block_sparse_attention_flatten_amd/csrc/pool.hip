// Block average pooling of Q and K ("NABLA: Neighborhood Adaptive Block-Level
// Attention", gist.science, Methodology: downsampling; lsdiaocha.cn article,
// sec. 2 step 1): the delegate of a block is the mean of its valid tokens.
//
// HBM-bound streaming read.  One wavefront pools one block: its 64 token rows
// are read as 16-byte chunks (a row of d elements spans L = d*elem/16 lanes,
// 64/L rows per load instruction), every load of the block is issued before
// any arithmetic, lanes accumulate in float32, and the 64/L row groups are
// folded with cross-lane shuffles.  Both the natural and the blocked layout
// are addressed in 8-token patch rows, so the reorder costs no extra pass.
#include "nabla_common.hpp"

namespace nabla {

namespace {

template <typename T, int D>
struct PoolShape {
  static constexpr int kElems = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int kLanesPerRow = D / kElems;         // 8, 16 or 32
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = kN / kRowsPerLoad;
};

template <typename T>
__device__ inline void accumulate(float* acc, const u32x4& raw);

template <>
__device__ inline void accumulate<__bf16>(float* acc, const u32x4& raw) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc[2 * w + 0] += __uint_as_float(raw[w] << 16);
    acc[2 * w + 1] += __uint_as_float(raw[w] & 0xffff0000u);
  }
}

template <>
__device__ inline void accumulate<float>(float* acc, const u32x4& raw) {
#pragma unroll
  for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[w]);
}

template <typename T, int D>
__global__ void __launch_bounds__(256) pool_kernel(const Geo g, const T* __restrict__ q,
                                                   const T* __restrict__ k,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar) {
  using S = PoolShape<T, D>;
  const int lane = threadIdx.x & 63;
  const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (head, block)
  if (gb >= g.bh * g.nb) return;
  const int64_t head = gb / g.nb;
  const int b = (int)(gb - head * g.nb);
  const T* x = blockIdx.y == 0 ? q : k;
  float* out = blockIdx.y == 0 ? qbar : kbar;

  const BlockCoord bc = block_coord(g, b);
  const int rv = block_rows_valid(g, bc);
  const int cv = block_cols_valid(g, bc);
  const T* base = x + head * (int64_t)g.head_elems + block_base(g, b, bc);
  const int row_step = block_row_step(g);
  const int chunk = lane % S::kLanesPerRow;
  const int row0 = lane / S::kLanesPerRow;

  u32x4 raw[S::kLoads];
#pragma unroll
  for (int it = 0; it < S::kLoads; ++it) {
    const int s = row0 + it * S::kRowsPerLoad;            // slot in the block
    const int i = s >> 3, j = s & 7;
    if (i < rv && j < cv) {
      raw[it] = *(const u32x4*)(base + i * row_step + j * D + chunk * S::kElems);
    } else {
      raw[it] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  float acc[S::kElems];
#pragma unroll
  for (int e = 0; e < S::kElems; ++e) acc[e] = 0.f;
#pragma unroll
  for (int it = 0; it < S::kLoads; ++it) accumulate<T>(acc, raw[it]);
#pragma unroll
  for (int off = S::kLanesPerRow; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < S::kElems; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (lane < S::kLanesPerRow) {
    const float cnt = (float)(rv * cv);
    float* dst = out + gb * D + chunk * S::kElems;
#pragma unroll
    for (int e = 0; e < S::kElems; e += 4) {
      f32x4 v = {acc[e] / cnt, acc[e + 1] / cnt, acc[e + 2] / cnt, acc[e + 3] / cnt};
      *(f32x4*)(dst + e) = v;
    }
  }
}

template <typename T, int D>
hipError_t launch(const Geo& g, const void* q, const void* k, float* qbar, float* kbar,
                  hipStream_t s) {
  const int64_t waves = g.bh * g.nb;
  const dim3 grid((unsigned)((waves + 3) / 4), 2);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, s, g, (const T*)q, (const T*)k,
                     qbar, kbar);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Geo& g, bool bf16, const void* q, const void* k, float* qbar,
                       float* kbar, hipStream_t s) {
  if (bf16) {
    return g.d == 64 ? launch<__bf16, 64>(g, q, k, qbar, kbar, s)
                     : launch<__bf16, 128>(g, q, k, qbar, kbar, s);
  }
  return g.d == 64 ? launch<float, 64>(g, q, k, qbar, kbar, s)
                   : launch<float, 128>(g, q, k, qbar, kbar, s);
}

}  // namespace nabla
