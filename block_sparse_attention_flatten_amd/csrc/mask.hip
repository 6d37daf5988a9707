// Adaptive block mask ("NABLA: Neighborhood Adaptive Block-Level Attention",
// gist.science, Methodology: reduced attention, CDF thresholding, hybrid
// integration with STA; lsdiaocha.cn article, sec. 2 step 2 and sec. 4).
//
// One workgroup of R wavefronts handles R = 16 (or 8) consecutive
// query-block rows of one head (the R x nb score tile fills up to ~80 KB of
// LDS, so one wavefront per row keeps several wavefronts per SIMD busy):
//   1. scores s[r][c] = qbar_r . kbar_c / sqrt(d) for all c, on fp32 matrix
//      cores (v_mfma_f32_16x16x4f32), staged in LDS;
//   2. one wavefront per row: softmax numerators e_c = exp(s_c - max) in
//      float32, Z = sum e, then the CDF cut.  Sorting the row is not needed to
//      find the kept set: it is exactly {c : e_c > v*} plus the lowest-index
//      blocks with e_c == v* that are needed to reach thr*Z, where v* is the
//      largest float with sum_{e_c >= v*} e_c >= thr*Z.  v* is found bit by bit
//      on the IEEE pattern (31 steps of a masked wavefront sum; the partial
//      sums use one fixed summation tree, so they are monotone in v and the
//      search is exact).  This is the same set as "sort descending, keep until
//      the cumulative mass reaches thr" (ties: lower index first);
//   3. the STA window (clipped box in block coordinates) is OR-ed into the
//      row's bit words, which are written with the row count.
#include "nabla_common.hpp"

namespace nabla {

namespace {

// Wavefront reductions on the DPP network (no LDS round trips): row-local
// butterflies leave every lane of a 16-lane row holding the row's result,
// row_bcast:15 / row_bcast:31 fold the rows into lane 63, which is read out
// as a wavefront-uniform value.
template <int kCtrl, int kRowMask, typename T>
__device__ inline T dpp_src(T x) {
  return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl,
                                                           kRowMask, 0xF, false));
}
template <typename T, typename Op>
__device__ inline T wave_reduce(T x, Op op) {
  x = op(x, dpp_src<0xB1, 0xF>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp_src<0x4E, 0xF>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp_src<0x141, 0xF>(x));   // row_half_mirror
  x = op(x, dpp_src<0x140, 0xF>(x));   // row_mirror
  x = op(x, dpp_src<0x142, 0xA>(x));   // row_bcast:15 -> rows 1, 3
  x = op(x, dpp_src<0x143, 0xC>(x));   // row_bcast:31 -> rows 2, 3
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ inline float wave_sum(float x) {
  return wave_reduce(x, [](float a, float b) { return a + b; });
}
__device__ inline int wave_sum_i(int x) {
  return wave_reduce(x, [](int a, int b) { return a + b; });
}
// For the max, rows a row_bcast step does not write must see the identity
// (-inf) rather than 0: it comes in through the DPP `old` operand.
template <int kCtrl, int kRowMask>
__device__ inline float dpp_src_max(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, -INFINITY),
                                                        __builtin_bit_cast(int, x), kCtrl,
                                                        kRowMask, 0xF, false));
}
__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp_src_max<0xB1, 0xF>(x));
  x = fmaxf(x, dpp_src_max<0x4E, 0xF>(x));
  x = fmaxf(x, dpp_src_max<0x141, 0xF>(x));
  x = fmaxf(x, dpp_src_max<0x140, 0xF>(x));
  x = fmaxf(x, dpp_src_max<0x142, 0xA>(x));
  x = fmaxf(x, dpp_src_max<0x143, 0xC>(x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Bits of word `w` (blocks 32w .. 32w+31) that fall inside the STA box around
// block (t, hb, wb), box half-widths (rt, rh, rw), clipped at the grid borders.
__device__ inline uint32_t sta_word(const Geo& g, int w, int t, int hb, int wb, int rt, int rh,
                                    int rw) {
  uint32_t bits = 0;
  const int lo_w = wb - rw < 0 ? 0 : wb - rw;
  const int hi_w = wb + rw >= g.gw ? g.gw - 1 : wb + rw;
  const int w0 = 32 * w, w1 = 32 * w + 31;
  for (int tt = t - rt; tt <= t + rt; ++tt) {
    if (tt < 0 || tt >= g.T) continue;
    for (int hh = hb - rh; hh <= hb + rh; ++hh) {
      if (hh < 0 || hh >= g.gh) continue;
      const int first = (tt * g.gh + hh) * g.gw + lo_w;    // a contiguous run of blocks
      const int last = (tt * g.gh + hh) * g.gw + hi_w;
      const int a = first > w0 ? first : w0;
      const int b = last < w1 ? last : w1;
      if (a <= b) {
        const int n = b - a + 1;
        const uint32_t run = n == 32 ? 0xffffffffu : ((1u << n) - 1u);
        bits |= run << (a - w0);
      }
    }
  }
  return bits;
}

// One wavefront per row of the workgroup's R rows (R * 64 threads).
template <int D, int R, int J>
__global__ void __launch_bounds__(R * 64) mask_kernel(const Geo g, const float* __restrict__ qbar,
                                                   const float* __restrict__ kbar, float scale,
                                                   float thr, int rt, int rh, int rw,
                                                   uint32_t* __restrict__ bits,
                                                   int32_t* __restrict__ count,
                                                   uint32_t* __restrict__ abits, int lds_stride) {
  extern __shared__ float S[];   // [R][lds_stride] scores in the exp2 domain
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  const int64_t head = blockIdx.y;
  const int r0 = blockIdx.x * R;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float* Qh = qbar + head * nb * D;
  const float* Kh = kbar + head * nb * D;

  // ---- 1. scores on fp32 matrix cores: C[16 rows][16 cols] per tile ----
  {
    const int i16 = lane & 15;          // A row / B column handled by this lane
    const int g4 = lane >> 4;           // k sub-index
    // The contraction index is permuted consistently for A and B: in step
    // 4t+u this lane supplies element 16t + 4*g4 + u of its row.
    f32x4 a[D / 16];
    const int qrow = r0 + i16;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      a[t] = (i16 < R && qrow < nb) ? *(const f32x4*)(Qh + (int64_t)qrow * D + 16 * t + 4 * g4)
                                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int ntiles = (nb + 15) >> 4;
    for (int ct = wave; ct < ntiles; ct += R) {
      const int col = ct * 16 + i16;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      f32x4 bv[D / 16];
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        bv[t] = col < nb ? *(const f32x4*)(Kh + (int64_t)col * D + 16 * t + 4 * g4)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t][u], bv[t][u], acc, 0, 0, 0);
        }
      }
      // acc[r] = C[4*g4 + r][i16]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g4 + r;
        if (row < R) S[row * lds_stride + ct * 16 + i16] = acc[r] * scale;
      }
    }
  }
  __syncthreads();

  // ---- 2./3. one wavefront per row: softmax numerators, CDF cut, STA ----
  const int pf = g.gh * g.gw;
  for (int ri = wave; ri < R; ri += R) {
    const int row = r0 + ri;
    if (row >= nb) break;
    const float* srow = S + ri * lds_stride;
    float e[J];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      e[j] = c < nb ? srow[c] : -INFINITY;
      mx = fmaxf(mx, e[j]);
    }
    mx = wave_max(mx);
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      e[j] = c < nb ? __builtin_amdgcn_exp2f(e[j] - mx) : 0.f;
      part += e[j];
    }
    const float Z = wave_sum(part);

    // kept-set words: lane w holds words w and w + 64
    uint32_t kw0 = 0, kw1 = 0;
    if (thr <= 0.0f) {
      // adaptive part off (pure STA): nothing kept here
    } else if (thr >= 1.0f) {
      for (int w = lane; w < nw; w += 64) {
        const int n = nb - 32 * w;
        const uint32_t v = n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
        if (w < 64) kw0 = v; else kw1 = v;
      }
    } else {
      const float target = thr * Z;
      uint32_t v = 0;
      for (int bit = 30; bit >= 0; --bit) {
        const uint32_t cand = v | (1u << bit);
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) p += __float_as_uint(e[j]) >= cand ? e[j] : 0.f;
        if (wave_sum(p) >= target) v = cand;
      }
      // mass strictly above v*, and how many ties at v* are needed
      float above = 0.f;
      int nties = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t u = __float_as_uint(e[j]);
        above += u > v ? e[j] : 0.f;
        nties += u == v ? 1 : 0;
      }
      float acc = wave_sum(above);
      nties = wave_sum_i(nties);
      const float vf = __uint_as_float(v);
      int need = 0;
      while (need < nties && acc < target) {
        acc += vf;
        ++need;
      }
      if (need == 0) need = 0;   // the mass above v* already reaches thr only if no tie is needed
      int rank_base = 0;         // ties ranked by block index (j-major, then lane)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const uint32_t u = __float_as_uint(e[j]);
        const int c = lane + 64 * j;
        const bool tie = c < nb && u == v;
        const uint64_t tb = __ballot(tie);
        const int rank = rank_base + __popcll(tb & ((1ull << lane) - 1ull));
        const bool keep = c < nb && (u > v || (tie && rank < need));
        const uint64_t kb = __ballot(keep);
        rank_base += __popcll(tb);
        const uint32_t lo = (uint32_t)kb, hi = (uint32_t)(kb >> 32);
        if (2 * j < 64) {
          if (lane == 2 * j) kw0 = lo;
          if (lane == 2 * j + 1) kw0 = hi;
        } else {
          if (lane == 2 * j - 64) kw1 = lo;
          if (lane == 2 * j - 63) kw1 = hi;
        }
      }
    }

    const int64_t obase = (head * nb + row) * (int64_t)nw;
    if (abits != nullptr) {
      if (lane < nw) abits[obase + lane] = kw0;
      if (lane + 64 < nw) abits[obase + lane + 64] = kw1;
    }
    if (rt >= 0) {
      const int t = row / pf;
      const int rem = row - t * pf;
      const int hb = rem / g.gw;
      const int wb = rem - hb * g.gw;
      if (lane < nw) kw0 |= sta_word(g, lane, t, hb, wb, rt, rh, rw);
      if (lane + 64 < nw) kw1 |= sta_word(g, lane + 64, t, hb, wb, rt, rh, rw);
    }
    if (lane < nw) bits[obase + lane] = kw0;
    if (lane + 64 < nw) bits[obase + lane + 64] = kw1;
    const int cnt = wave_sum_i(__popc(kw0) + __popc(kw1));
    if (lane == 0) count[head * nb + row] = cnt;
  }
}

template <int D, int R, int J>
hipError_t launch_t(const Geo& g, const float* qbar, const float* kbar, float thr, int rt, int rh,
                    int rw, uint32_t* bits, int32_t* cnt, uint32_t* abits, hipStream_t s) {
  // row stride in floats: >= nb, and = 16 (mod 32) so the 4 rows a wavefront
  // writes per tile land on alternating halves of the 32 LDS banks
  int stride = ((g.nb + 15) / 16) * 16;
  if (stride % 32 == 0) stride += 16;
  const size_t lds = (size_t)R * stride * sizeof(float);
  auto kern = mask_kernel<D, R, J>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nb + R - 1) / R, (unsigned)g.bh);
  // scores q.k / sqrt(d), carried in the exp2 domain (times log2 e), so the
  // softmax numerators are exp2(s - max)
  const float scale = 1.4426950408889634f / sqrtf((float)D);
  hipLaunchKernelGGL(kern, grid, dim3(R * 64), lds, s, g, qbar, kbar, scale, thr, rt, rh, rw, bits,
                     cnt, abits, stride);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Geo& g, const float* qbar, const float* kbar, float thr, int rt, int rh,
                    int rw, uint32_t* bits, int32_t* cnt, uint32_t* abits, hipStream_t s) {
  const int nb = g.nb;
  if (nb <= 256) return launch_t<D, 16, 4>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 512) return launch_t<D, 16, 8>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 1024) return launch_t<D, 16, 16>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 1280) return launch_t<D, 16, 20>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 1536) return launch_t<D, 16, 24>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 2048) return launch_t<D, 16, 32>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 2496) return launch_t<D, 16, 39>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  if (nb <= 3072) return launch_t<D, 8, 48>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
  return launch_t<D, 8, 64>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
}

}  // namespace

hipError_t launch_mask(const Geo& g, const float* qbar, const float* kbar, float thr,
                       const int sta[3], uint32_t* bits, int32_t* cnt, uint32_t* abits,
                       hipStream_t s) {
  // STA half-widths; rt < 0 switches the window off
  int rt = -1, rh = -1, rw = -1;
  if (sta[0] > 0) {
    rt = sta[0] / 2;
    rh = sta[1] / 2;
    rw = sta[2] / 2;
  }
  return g.d == 64 ? launch_d<64>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s)
                   : launch_d<128>(g, qbar, kbar, thr, rt, rh, rw, bits, cnt, abits, s);
}

}  // namespace nabla
