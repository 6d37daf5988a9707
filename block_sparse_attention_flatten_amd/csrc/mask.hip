// Adaptive block mask ("NABLA: Neighborhood Adaptive Block-Level Attention",
// gist.science, Methodology: reduced attention, CDF thresholding, hybrid
// integration with STA; lsdiaocha.cn article, sec. 2 step 2 and sec. 4), as a
// standalone call on pooled inputs (nabla_mask) and as the middle step of
// the mask construction call (nabla_mask_build: pooling, mask, lists).
//
// A row group is R rows of one head: their scores (float32 accuracy from
// split bf16 products on the matrix cores) staged in an LDS tile
// (score_tiles), then one wavefront per row for
// softmax, CDF cut and STA union (cut_rows); see mask_items.hpp.
//
// The mask construction call runs pooling, mask and compaction as three
// launches in order on one stream: every dependency (a head's mask needs all
// of its pooled keys, a list needs the row counts of all earlier rows) then
// crosses a kernel boundary, which is where writes made through one XCD's L2
// become visible to the others.
#include "mask_items.hpp"

namespace nabla {

namespace {

using namespace mask_detail;

template <int D, int R, int NW, int J>
__global__ void __launch_bounds__(NW * 64, 4) mask_kernel(const Geo g, const MaskArgs a) {
  extern __shared__ float S[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  score_tiles<D, R>(g, a, blockIdx.y, blockIdx.x * R, S, wave, NW, blockIdx.x);
  __syncthreads();
  cut_rows<J>(g, a, blockIdx.y, blockIdx.x * R, R, S, wave, NW);
}

template <int D, int R, int NW, int J>
hipError_t mask_t(const Geo& g, MaskArgs a, hipStream_t s) {
  a.stride = mask_stride(g.nb);
  const size_t lds = (size_t)R * a.stride * sizeof(float);
  auto kern = mask_kernel<D, R, NW, J>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const dim3 grid((g.nb + R - 1) / R, (unsigned)g.bh);
  hipLaunchKernelGGL(kern, grid, dim3(NW * 64), lds, s, g, a);
  return hipGetLastError();
}

// Row-group shape of the standalone mask kernel by the number of blocks per
// head: R rows per group (the R x nb float32 score tile must fit LDS), NW
// wavefronts, J = ceil(nb / 64) row values per lane.  Up to nb = 1264 two
// 16-row groups fit a CU; above that a 16-row tile leaves room for one group
// per CU, whose score and cut phases then never overlap, and 8-row groups
// (two or more per CU, at twice the pooled-key reads) are faster: 1.66 vs
// 1.70 ms for the 2460-block mask construction, while at 1260 blocks 8-row
// groups lose (0.65 vs 0.57 ms).
template <int D, typename F>
hipError_t dispatch_shape(int nb, const F& f) {
  if (nb <= 256) return f.template operator()<D, 16, 8, 4>();
  if (nb <= 512) return f.template operator()<D, 16, 8, 8>();
  if (nb <= 1024) return f.template operator()<D, 16, 8, 16>();
  if (nb <= 1280) return f.template operator()<D, 16, 8, 20>();
  if (nb <= 1536) return f.template operator()<D, 8, 8, 24>();
  if (nb <= 2048) return f.template operator()<D, 8, 8, 32>();
  if (nb <= 2496) return f.template operator()<D, 8, 8, 39>();
  if (nb <= 3072) return f.template operator()<D, 8, 8, 48>();
  return f.template operator()<D, 8, 8, 64>();
}

MaskArgs mask_args(const Geo& g, const float* qbar, const __bf16* kbar, float thr,
                   const int sta[3], uint32_t* bits, int32_t* cnt, uint32_t* abits) {
  MaskArgs a;
  a.qbar = qbar;
  a.kbar = kbar;
  // scores q.k / sqrt(d), carried in the exp2 domain (times log2 e), so the
  // softmax numerators are exp2(s - max)
  a.scale = 1.4426950408889634f / sqrtf((float)g.d);
  a.thr = thr;
  a.rt = a.rh = a.rw = -1;           // STA half-widths; rt < 0 switches the window off
  if (sta[0] > 0) {
    a.rt = sta[0] / 2;
    a.rh = sta[1] / 2;
    a.rw = sta[2] / 2;
  }
  a.bits = bits;
  a.count = cnt;
  a.abits = abits;
  a.stride = 0;
  return a;
}

struct MaskRun {
  const Geo& g;
  const MaskArgs& a;
  hipStream_t s;
  template <int D, int R, int NW, int J>
  hipError_t operator()() const { return mask_t<D, R, NW, J>(g, a, s); }
};

}  // namespace

hipError_t launch_mask(const Geo& g, const float* qbar, const __bf16* kbar, float thr,
                       const int sta[3], uint32_t* bits, int32_t* cnt, uint32_t* abits,
                       hipStream_t s) {
  const MaskArgs a = mask_args(g, qbar, kbar, thr, sta, bits, cnt, abits);
  const MaskRun run{g, a, s};
  return g.d == 64 ? dispatch_shape<64>(g.nb, run) : dispatch_shape<128>(g.nb, run);
}

hipError_t launch_mask_build(const Geo& g, bool bf16, const void* q, const void* k, float* qbar,
                             __bf16* kbar, float thr, const int sta[3], uint32_t* bits,
                             int32_t* cnt, uint32_t* abits, int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t s) {
  hipError_t e = launch_pool(g, bf16, q, k, qbar, kbar, s);
  if (e == hipSuccess) e = launch_mask(g, qbar, kbar, thr, sta, bits, cnt, abits, s);
  if (e == hipSuccess) e = launch_compact(g, bits, cnt, row_ptr, col_idx, s);
  return e;
}

}  // namespace nabla
