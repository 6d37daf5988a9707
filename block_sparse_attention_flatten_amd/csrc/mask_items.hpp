// Device-side pieces of mask construction, each the work of one wavefront,
// used by the pooling, mask and compaction kernels (pool.hip, mask.hip,
// compact.hip) and, for the summation order of the means, by the layout pass
// after a QKV projection (qkv_split.hip):
//   * pool_block  - the mean of one block's valid tokens ("NABLA:
//     Neighborhood Adaptive Block-Level Attention", gist.science,
//     Methodology: downsampling);
//   * score_tiles / cut_rows - a group of R rows of one head: reduced scores
//     (float32 accuracy from split bf16 products) staged in LDS, then
//     softmax, CDF cut and STA union per row (Methodology: reduced attention,
//     CDF thresholding, hybrid integration with STA);
//   * compact_rows - rows of a mask expanded into the compressed kept lists
//     (lsdiaocha.cn article on NABLA, sec. 5: compressed sparse storage).
// Because each piece is one wavefront's work, a kernel may hand the pieces to
// its wavefronts in any way and still produce the same bits.
#pragma once

#include <type_traits>

#include "nabla_common.hpp"

namespace nabla {
namespace mask_detail {

// ---------------------------------------------------------------------------
// wavefront reductions on the DPP network: row-local butterflies, then
// row_bcast:15 / row_bcast:31 fold the four rows into lane 63, read out as a
// wavefront-uniform value.  Rows a step does not write keep `old`, which
// carries the identity of the operation.
// ---------------------------------------------------------------------------
template <int kCtrl, int kRowMask>
__device__ inline uint32_t dpp_u(uint32_t x, uint32_t ident) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)ident, (int)x, kCtrl, kRowMask, 0xF, false);
}
template <typename Op>
__device__ inline uint32_t wave_reduce_u(uint32_t x, uint32_t ident, Op op) {
  x = op(x, dpp_u<0xB1, 0xF>(x, ident));    // quad_perm [1,0,3,2]
  x = op(x, dpp_u<0x4E, 0xF>(x, ident));    // quad_perm [2,3,0,1]
  x = op(x, dpp_u<0x141, 0xF>(x, ident));   // row_half_mirror
  x = op(x, dpp_u<0x140, 0xF>(x, ident));   // row_mirror
  x = op(x, dpp_u<0x142, 0xA>(x, ident));   // row_bcast:15 -> rows 1, 3
  x = op(x, dpp_u<0x143, 0xC>(x, ident));   // row_bcast:31 -> rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ inline float wave_sum(float x) {
  return __uint_as_float(wave_reduce_u(__float_as_uint(x), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ inline int wave_sum_i(int x) {
  return (int)wave_reduce_u((uint32_t)x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}
__device__ inline float wave_max(float x) {
  return __uint_as_float(wave_reduce_u(__float_as_uint(x), __float_as_uint(-INFINITY),
                                       [](uint32_t a, uint32_t b) {
                                         return __float_as_uint(
                                             fmaxf(__uint_as_float(a), __uint_as_float(b)));
                                       }));
}
__device__ inline uint32_t wave_max_u(uint32_t x) {
  return wave_reduce_u(x, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ inline uint32_t wave_min_u(uint32_t x) {
  return wave_reduce_u(x, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
// number of set bits of `b` below this lane
__device__ inline int lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// ---------------------------------------------------------------------------
// block pooling: one wavefront reads the block's 64 token rows as 16-byte
// chunks (a row of d elements spans L = d * elem / 16 lanes, 64 / L rows per
// load), issues every load before any arithmetic, accumulates in float32 and
// folds the row groups with cross-lane shuffles.  Pad rows and columns are
// skipped; the mean is over the valid tokens.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct PoolShape {
  static constexpr int kElems = 16 / sizeof(T);          // elements per 16-byte chunk
  static constexpr int kLanesPerRow = D / kElems;         // 8, 16 or 32
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = kN / kRowsPerLoad;
};

// acc[e] += element e of the 16-byte chunk (bf16: a shift or a mask makes
// each half a float32).
template <typename T>
__device__ inline void pool_accumulate(float* acc, const u32x4& raw);
template <>
__device__ inline void pool_accumulate<__bf16>(float* acc, const u32x4& raw) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    acc[2 * w + 0] += __uint_as_float(raw[w] << 16);
    acc[2 * w + 1] += __uint_as_float(raw[w] & 0xffff0000u);
  }
}
template <>
__device__ inline void pool_accumulate<float>(float* acc, const u32x4& raw) {
#pragma unroll
  for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[w]);
}

// Mean of block b of one head (x: the head's tensor in geom's layout).
// Lanes 0 .. kLanesPerRow - 1 receive elements chunk * kElems .. + kElems - 1
// of the mean (chunk = lane); the other lanes hold partial sums.
//
// The block is read through a buffer descriptor that ends at its last valid
// token, so pad rows (past the end) load zeros; pad columns get a lane
// offset past the end as well.  Every load is issued unconditionally, in
// groups of at most 16 (64 registers), and the accumulation order is fixed.
// Slot s = row0 + kRowsPerLoad * it of the block is patch row it / P, patch
// column row0 + kRowsPerLoad * (it % P), P = 8 / kRowsPerLoad, so a lane needs
// P offsets and the patch row goes into the scalar offset.
template <typename T, int D>
__device__ inline void pool_block(const Geo& g, const T* x, int b,
                                  float (&mean)[PoolShape<T, D>::kElems]) {
  using S = PoolShape<T, D>;
  constexpr int P = kP / S::kRowsPerLoad;           // loads per patch row
  constexpr int kRowsPerGroup = 16 / P < kP ? 16 / P : kP;
  const int lane = threadIdx.x & 63;
  const BlockCoord bc = block_coord(g, b);
  const int rv = block_rows_valid(g, bc);
  const int cv = block_cols_valid(g, bc);
  const int row_step = block_row_step(g);
  const __amdgpu_buffer_rsrc_t rs =
      buffer_rsrc(x + block_base(g, b, bc), (uint32_t)(((rv - 1) * row_step + cv * D) * sizeof(T)));
  const int chunk = lane % S::kLanesPerRow;
  const int row0 = lane / S::kLanesPerRow;
  uint32_t voff[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = row0 + S::kRowsPerLoad * p;       // patch column
    voff[p] = j < cv ? (uint32_t)((j * D + chunk * S::kElems) * sizeof(T)) : 0x80000000u;
  }
#pragma unroll
  for (int e = 0; e < S::kElems; ++e) mean[e] = 0.f;
#pragma unroll
  for (int i0 = 0; i0 < kP; i0 += kRowsPerGroup) {
    u32x4 raw[kRowsPerGroup * P];
#pragma unroll
    for (int r = 0; r < kRowsPerGroup; ++r)
#pragma unroll
      for (int p = 0; p < P; ++p)
        raw[r * P + p] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, voff[p],
            (uint32_t)__builtin_amdgcn_readfirstlane((int)((i0 + r) * row_step * sizeof(T))), 0);
#pragma unroll
    for (int it = 0; it < kRowsPerGroup * P; ++it) pool_accumulate<T>(mean, raw[it]);
  }
#pragma unroll
  for (int off = S::kLanesPerRow; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < S::kElems; ++e) mean[e] += __shfl_xor(mean[e], off);
  }
  const float inv = 1.0f / (float)(rv * cv);    // exact for the 64 slots of a full block
#pragma unroll
  for (int e = 0; e < S::kElems; ++e) mean[e] *= inv;
}

// Store pool_block's result as row `row` of a head's pooled keys: each mean
// as its three exact bf16 parts, in the tiled order of kbar_offset (the
// lane's kElems consecutive channels are consecutive there).
__device__ inline void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
  h = (__bf16)x;
  const float r = x - (float)h;     // exact
  m = (__bf16)r;
  l = (__bf16)(r - (float)m);       // exact, and exactly a bf16
}
template <typename T, int D>
__device__ inline void store_mean_tiled(const float (&mean)[PoolShape<T, D>::kElems],
                                        __bf16* head_base, int row) {
  using S = PoolShape<T, D>;
  constexpr int E = S::kElems;
  typedef __attribute__((ext_vector_type(E))) __bf16 part_t;
  const int lane = threadIdx.x & 63;
  if (lane < S::kLanesPerRow) {
    part_t h, m, l;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      __bf16 a, b, c;
      split3(mean[e], a, b, c);
      h[e] = a;
      m[e] = b;
      l[e] = c;
    }
    const int c0 = lane * E;
    *(part_t*)(head_base + kbar_offset(row, c0, 0, D)) = h;
    *(part_t*)(head_base + kbar_offset(row, c0, 1, D)) = m;
    *(part_t*)(head_base + kbar_offset(row, c0, 2, D)) = l;
  }
}

// Store pool_block's result to dst[0 .. D) (global or LDS).
template <typename T, int D>
__device__ inline void store_mean(const float (&mean)[PoolShape<T, D>::kElems], float* dst) {
  using S = PoolShape<T, D>;
  const int lane = threadIdx.x & 63;
  if (lane < S::kLanesPerRow) {
#pragma unroll
    for (int e = 0; e < S::kElems; e += 4)
      *(f32x4*)(dst + lane * S::kElems + e) =
          f32x4{mean[e], mean[e + 1], mean[e + 2], mean[e + 3]};
  }
}

// ---------------------------------------------------------------------------
// STA window: OR the clipped box of half-widths (rt, rh, rw) around block
// (t, hb, wb) into a row's words in LDS.  The box is (2rt+1)(2rh+1)
// contiguous runs of blocks; each run touches one or two words.  The run
// bounds are wavefront-uniform; one lane applies them.
// ---------------------------------------------------------------------------
__device__ inline void sta_or(const Geo& g, int t, int hb, int wb, int rt, int rh, int rw,
                              uint32_t* words) {
  const int lane = threadIdx.x & 63;
  const int lo_w = wb - rw < 0 ? 0 : wb - rw;
  const int hi_w = wb + rw >= g.gw ? g.gw - 1 : wb + rw;
  const int t0 = t - rt < 0 ? 0 : t - rt, t1 = t + rt >= g.T ? g.T - 1 : t + rt;
  const int h0 = hb - rh < 0 ? 0 : hb - rh, h1 = hb + rh >= g.gh ? g.gh - 1 : hb + rh;
  for (int tt = t0; tt <= t1; ++tt) {
    for (int hh = h0; hh <= h1; ++hh) {
      const int first = (tt * g.gh + hh) * g.gw + lo_w;
      const int last = (tt * g.gh + hh) * g.gw + hi_w;
      for (int w = first >> 5; w <= (last >> 5); ++w) {
        const int a = first > 32 * w ? first : 32 * w;
        const int b = last < 32 * w + 31 ? last : 32 * w + 31;
        const int n = b - a + 1;
        const uint32_t m = (n == 32 ? 0xffffffffu : ((1u << n) - 1u)) << (a - 32 * w);
        if (lane == 0) atomicOr(&words[w], m);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// CDF cut of one row, one wavefront.
//
// With e_c = exp2(s_c - max) and Z = sum e, the kept set of "sort descending,
// keep until the cumulative mass reaches thr" (ties: lower index first) is
// {c : e_c > v*} plus the lowest-index blocks with e_c = v* needed to reach
// thr * Z, where v* is the largest value v with F(v) = sum_{e_c >= v} e_c >=
// thr * Z.  v* is always one of the e_c, and since e_c >= 0 comparing IEEE
// bit patterns as integers compares the values.  v* is found as a radix
// select on the bit pattern, narrowing the candidate set as it goes:
//   1. exponent: bisection over the binades between the row's smallest e
//      (from the smallest score) and 1 (the max is exactly 1), each step a
//      masked sum over the row;
//   2. the elements of the chosen binade are compacted into LDS (the row's
//      own score area, no longer needed); bisection over mantissa bits
//      22..15 on those candidates, held in registers when there are at most
//      256 of them, with the mass above the binade added;
//   3. the candidates that share those bits are compacted again (usually a
//      handful) and v* is the largest of them whose F still reaches the
//      target, F evaluated for every candidate at once.
// The mass above each level's range is the sum of the last failing test of
// the level before (a binary search ends next to its last failure), or of
// the level before that if none failed.  Every F is a sum of non-negative
// terms in one fixed order, so it is non-increasing in v and each search is
// exact for the sums it evaluates.  The levels sum in different orders, so
// where the crossing lies within float32 rounding of thr * Z the chosen cut
// is one of the cuts that are correct to that rounding.
//
// e: this lane's values (block c = lane + 64 j; 0 for c >= nb);
// xlo: the smallest exponent (s_c - max) of the row; cand: LDS scratch of
// >= nb floats owned by this wavefront, which on return holds the row's kept
// words (ceil(nb / 32) of them; block c is bit c % 32 of word c / 32).
// ---------------------------------------------------------------------------
template <int J>
__device__ inline void cdf_cut(const float (&e)[J], float xlo, int nb, float Z, float thr,
                               float* cand) {
  const int lane = threadIdx.x & 63;
  const int nw = (nb + 31) >> 5;
  uint32_t* words = (uint32_t*)cand;
  if (thr <= 0.0f || thr >= 1.0f) {
    // thr = 0: the adaptive part is off (pure STA), nothing kept here;
    // thr = 1: every block is kept
    for (int w = lane; w < nw; w += 64) {
      const int n = nb - 32 * w;
      words[w] = thr <= 0.0f ? 0u : (n >= 32 ? 0xffffffffu : ((1u << n) - 1u));
    }
    return;
  }
  const float target = thr * Z;

  // ---- 1. binade of v*: largest E in [lo, 127] with F(2^(E-127)) >= target.
  // exp2(x) >= 2^floor(x) up to rounding, so no element lies below binade
  // floor(xlo) + 126, and F there is the whole row: Z >= target.
  // (Z is summed in the same two chains as these masked sums, so F at the
  // lower bound is exactly Z.)
  int lo = (int)floorf(xlo) + 126;
  lo = lo < 0 ? 0 : (lo > 127 ? 127 : lo);
  int hi = 127;                      // the row max is exactly 1.0
  float A1 = 0.f;                    // mass of the binades above the chosen one
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    const uint32_t c = (uint32_t)mid << 23;
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float x = __float_as_uint(e[j]) >= c ? e[j] : 0.f;
      if (j & 1) p1 += x; else p0 += x;
    }
    const float m = wave_sum(p0 + p1);
    if (m >= target) {
      lo = mid;
    } else {
      hi = mid - 1;
      A1 = m;
    }
  }

  // ---- 2. the binade's elements (zeros of pad slots too, when lo = 0: they
  // add nothing to any sum) into LDS; bisection over mantissa bits 22..15
  const uint32_t lo1 = (uint32_t)lo << 23;
  int ncand = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const bool in = __float_as_uint(e[j]) - lo1 < (1u << 23);
    const uint64_t b = __ballot(in);
    if (in) cand[ncand + lanes_below(b)] = e[j];
    ncand += __popcll(b);
  }
  uint32_t v = lo1;
  float A2 = A1;                     // mass above v's 17-bit prefix group
  if (ncand <= 256) {
    float c4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c4[k] = 64 * k + lane < ncand ? cand[64 * k + lane] : 0.f;
    for (int bit = 22; bit >= 15; --bit) {
      const uint32_t c = v | (1u << bit);
      float p = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) p += __float_as_uint(c4[k]) >= c ? c4[k] : 0.f;
      const float m = A1 + wave_sum(p);
      if (m >= target) v = c; else A2 = m;
    }
  } else {
    for (int bit = 22; bit >= 15; --bit) {
      const uint32_t c = v | (1u << bit);
      float p = 0.f;
      for (int i = lane; i < ncand; i += 64) {
        const float x = cand[i];
        p += __float_as_uint(x) >= c ? x : 0.f;
      }
      const float m = A1 + wave_sum(p);
      if (m >= target) v = c; else A2 = m;
    }
  }

  // ---- 3. compact again to the candidates sharing v's top 9 + 8 bits
  //         (in place: new positions never pass the ones still to be read)
  const uint32_t key = v >> 15;
  int n2 = 0;
  for (int base = 0; base < ncand; base += 64) {
    const int i = base + lane;
    const float x = i < ncand ? cand[i] : 0.f;
    const bool in = i < ncand && (__float_as_uint(x) >> 15) == key;
    const uint64_t b = __ballot(in);
    if (in) cand[n2 + lanes_below(b)] = x;
    n2 += __popcll(b);
  }
  uint32_t vstar;
  float above_star;
  int nties;
  if (n2 <= 64) {
    // every candidate at once: F(c_l) = A2 + sum_{m : c_m >= c_l} c_m
    const bool mine = lane < n2;
    const float x = mine ? cand[lane] : 0.f;
    const uint32_t u = __float_as_uint(x);
    float f = 0.f;
    for (int m = 0; m < n2; ++m) {
      const uint32_t um = (uint32_t)__builtin_amdgcn_readlane((int)u, m);
      f += um >= u ? __uint_as_float(um) : 0.f;
    }
    const bool ok = mine && A2 + f >= target;
    if (__ballot(ok) != 0ull) {
      vstar = wave_max_u(ok ? u : 0u);
    } else {                         // rounding only: keep the whole group
      vstar = wave_min_u(mine ? u : 0xffffffffu);
    }
    above_star = A2 + wave_sum(mine && u > vstar ? x : 0.f);
    nties = __popcll(__ballot(mine && u == vstar));
  } else {
    // a dense group (e.g. exact ties across the row): bisection on bits 14..0
    for (int bit = 14; bit >= 0; --bit) {
      const uint32_t c = v | (1u << bit);
      float p = 0.f;
      for (int i = lane; i < n2; i += 64) {
        const float x = cand[i];
        p += __float_as_uint(x) >= c ? x : 0.f;
      }
      if (A2 + wave_sum(p) >= target) v = c;
    }
    vstar = v;
    float pa = 0.f;
    int pt = 0;
    for (int i = lane; i < n2; i += 64) {
      const float x = cand[i];
      const uint32_t u = __float_as_uint(x);
      pa += u > vstar ? x : 0.f;
      pt += u == vstar ? 1 : 0;
    }
    above_star = A2 + wave_sum(pa);
    nties = wave_sum_i(pt);
  }
  // how many of the ties at v* (taken by block index) reach the target
  const float vf = __uint_as_float(vstar);
  float acc = above_star;
  int need = 0;
  while (need < nties && acc < target) {
    acc += vf;
    ++need;
  }

  // ---- kept words: e > v*, plus the first `need` ties by block index.  v*
  // is positive (the max, 1, carries mass), so pad slots (e = 0) never pass.
  // The ballot of values j is words 2j, 2j + 1, stored by one lane (the
  // words past nw are zeros and stay inside the row's area).
  uint64_t* w64 = (uint64_t*)cand;
  if (need == nties) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint64_t b = __ballot(__float_as_uint(e[j]) >= vstar);
      if (lane == 0) w64[j] = b;
    }
  } else if (need == 0) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint64_t b = __ballot(__float_as_uint(e[j]) > vstar);
      if (lane == 0) w64[j] = b;
    }
  } else {
    int rank_base = 0;               // ties ranked by block index (j-major, then lane)
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t u = __float_as_uint(e[j]);
      const bool tie = u == vstar;
      const uint64_t tb = __ballot(tie);
      const int rank = rank_base + lanes_below(tb);
      const uint64_t b = __ballot(u > vstar || (tie && rank < need));
      if (lane == 0) w64[j] = b;
      rank_base += __popcll(tb);
    }
  }
}

// ---------------------------------------------------------------------------
// row groups of the reduced map
// ---------------------------------------------------------------------------
struct MaskArgs {
  const float* qbar;    // [bh, nb, d]
  const __bf16* kbar;   // per head kbar_head_elems(nb, d): split parts, tiled
  float scale;          // log2(e) / sqrt(d): scores carried in the exp2 domain
  float thr;
  int rt, rh, rw;       // STA half-widths; rt < 0: no window
  uint32_t* bits;       // [bh, nb, nw] union mask
  int32_t* count;       // [bh, nb]
  uint32_t* abits;      // optional [bh, nb, nw] adaptive-only mask
  int stride;           // LDS row stride of the score tile, in floats
};

// LDS floats a mask item needs: the R x stride score tile.
__host__ __device__ inline int mask_item_lds_floats(int R, int stride) { return R * stride; }

// Row stride of the score tile: >= nb and = 16 (mod 32), so the 4 rows a
// wavefront writes per tile land on alternating halves of the banks.
__host__ __device__ inline int mask_stride(int nb) {
  int s = ((nb + 15) / 16) * 16;
  if (s % 32 == 0) s += 16;
  return s;
}

// Scores of one row group (rows r0 .. r0 + R - 1 of a head) for the column
// tiles ct = first, first + step, ... (16 key blocks each) into the LDS
// tile S (R x a.stride floats), scaled into the exp2 domain.  One wavefront.
//
// q.k in float32 accuracy on bf16 matrix cores: with q = qh + qm + ql and
// k = kh + km + kl the exact three-part splits of the float32 means, the
// products qh.kh, qh.km, qm.kh, qh.kl, qm.km and ql.kh are formed by
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in float32); the
// three dropped ones are below 2^-25 of |q_i k_i| each.  Two accumulators
// take alternate products, so consecutive matrix instructions do not wait on
// each other, and the order is fixed.
//
// The query parts are split once per group from the float32 rows; the key
// parts come pre-split in their tiled order (kbar_offset) through a buffer
// descriptor, each 16-byte-per-lane load one contiguous kilobyte.  The next
// tile's loads of a k-step are issued as soon as that k-step's products have
// read their operands, so up to a tile of loads is in flight.  The
// wavefront walks its tiles starting at position rot (mod their count):
// workgroups working on the same head at once then read different K rows
// instead of all hitting the same lines (and L2 channel) together.
template <int D, int R>
__device__ inline void score_tiles(const Geo& g, const MaskArgs& a, int64_t head, int r0,
                                   float* S, int first, int step, int rot) {
  constexpr int KT = D / 32;          // k-steps of 32 channels
  const int nb = g.nb;
  const int lane = threadIdx.x & 63;
  const __bf16* Kh = a.kbar + head * kbar_head_elems(nb, D);
  const float* Qh = a.qbar + head * nb * D;
  const int i16 = lane & 15;          // A row / B column of this lane
  const int g4 = lane >> 4;           // channel group of 8 within a k-step
  const int qrow = r0 + i16;
  const bool arow = i16 < R && qrow < nb;
  const int ntiles = (nb + 15) >> 4;
  if (first >= ntiles) return;

  // A operand: row i16's channels 32 t + 8 g4 .. + 7, as three parts
  bf16x8 ah[KT], am[KT], al[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) {
    const float* src = Qh + (int64_t)qrow * D + 32 * t + 8 * g4;
    const f32x4 x0 = arow ? *(const f32x4*)src : f32x4{0.f, 0.f, 0.f, 0.f};
    const f32x4 x1 = arow ? *(const f32x4*)(src + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, m, l;
      split3(e < 4 ? x0[e] : x1[e - 4], h, m, l);
      ah[t][e] = h;
      am[t][e] = m;
      al[t][e] = l;
    }
  }

  // B operand: k-step t of tile ct is 3 KB at ct * KT * 3 KB + t * 3 KB (one
  // kilobyte per part); lanes of rows past the last block load zeros
  const __amdgpu_buffer_rsrc_t krs =
      buffer_rsrc(Kh, (uint32_t)(kbar_head_elems(nb, D) * (int64_t)sizeof(__bf16)));
  const uint32_t lane_off = (uint32_t)(lane * 16);
  auto load_kstep = [&](int ct, int t, bf16x8 (&b)[3]) {
    const uint32_t voff = ct * 16 + i16 < nb ? lane_off : 0x80000000u;
    // the tile offset is wavefront-uniform; say so, or the compiler wraps
    // each load in a loop over the distinct values it thinks lanes hold
    const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(ct * KT * 3 * 1024);
#pragma unroll
    for (int p = 0; p < 3; ++p)
      b[p] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                            krs, voff + 1024u * (3 * t + p), soff, 0));
  };
  const int n = (ntiles - first + step - 1) / step;   // this wavefront's tiles
  const int i = rot % n;
  auto tile_at = [&](int k) {          // k-th tile of the rotated walk
    const int m = i + k;
    return first + step * (m >= n ? m - n : m);
  };
  bf16x8 kb[KT][3];
  {
    const int ct = tile_at(0);
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      load_kstep(ct, t, kb[t]);
      __builtin_amdgcn_sched_barrier(0);   // same load order as in the loop
    }
  }
  for (int k = 0; k < n; ++k) {
    const int ct = tile_at(k);
    // after the last tile, the loads repeat it (unused): the load count per
    // iteration stays fixed, so the waits before each k-step stay exact
    const int nxt = k + 1 < n ? tile_at(k + 1) : ct;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], kb[t][0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], kb[t][1], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[t], kb[t][0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], kb[t][2], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am[t], kb[t][1], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[t], kb[t][0], acc1, 0, 0, 0);
      load_kstep(nxt, t, kb[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // acc[r] = C[4*g4 + r][i16]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g4 + r;
      if (row < R) S[row * a.stride + ct * 16 + i16] = (acc0[r] + acc1[r]) * a.scale;
    }
  }
}

// Softmax numerators, CDF cut, STA union and outputs of the rows
// r0 + ri, ri = first, first + step, ... < R whose scores are in S.  One
// wavefront; each row's LDS area serves as the cut's scratch.
template <int J>
__device__ inline void cut_rows(const Geo& g, const MaskArgs& a, int64_t head, int r0, int R,
                                float* S, int first, int step) {
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  const int lane = threadIdx.x & 63;
  const int pf = g.gh * g.gw;
  for (int ri = first; ri < R; ri += step) {
    const int row = r0 + ri;
    if (row >= nb) break;
    float* srow = S + ri * a.stride;
    float e[J];
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = lane + 64 * j;
      const float x = c < nb ? srow[c] : 0.f;
      e[j] = c < nb ? x : -INFINITY;
      mx = fmaxf(mx, e[j]);
      mn = fminf(mn, c < nb ? x : INFINITY);
    }
    mx = wave_max(mx);
    mn = -wave_max(-mn);
    float part0 = 0.f, part1 = 0.f;      // two chains (even and odd j): the
#pragma unroll                           // cut's masked sums use the same order
    for (int j = 0; j < J; ++j) {
      e[j] = __builtin_amdgcn_exp2f(e[j] - mx);   // pad slots: exp2(-inf) = 0
      if (j & 1) part1 += e[j]; else part0 += e[j];
    }
    const float Z = wave_sum(part0 + part1);
    cdf_cut<J>(e, mn - mx, nb, Z, a.thr, srow);
    uint32_t* words = (uint32_t*)srow;   // the row's kept words, in LDS

    const int64_t obase = (head * nb + row) * (int64_t)nw;
    if (a.abits != nullptr) {
      if (lane < nw) a.abits[obase + lane] = words[lane];
      if (lane + 64 < nw) a.abits[obase + lane + 64] = words[lane + 64];
    }
    if (a.rt >= 0) {
      const int t = row / pf;
      const int rem = row - t * pf;
      const int hb = rem / g.gw;
      sta_or(g, t, hb, rem - hb * g.gw, a.rt, a.rh, a.rw, words);
    }
    const uint32_t w0 = lane < nw ? words[lane] : 0u;
    const uint32_t w1 = lane + 64 < nw ? words[lane + 64] : 0u;
    if (lane < nw) a.bits[obase + lane] = w0;
    if (lane + 64 < nw) a.bits[obase + lane + 64] = w1;
    const int cnt = wave_sum_i(__popc(w0) + __popc(w1));
    if (lane == 0) a.count[head * nb + row] = cnt;
  }
}

// ---------------------------------------------------------------------------
// compaction of rows r0 .. r0 + n - 1 (n <= kCompactRows) of one head by one
// wavefront: the counts of all earlier rows of the head give the start, a
// scan of the unit's own counts the row pointers.  Each row is expanded in
// chunks of 64 blocks: lane l holds chunk l of the row (nb <= 4096, so one
// 64-bit word per lane), a chunk read out with two readlanes IS the ballot of
// its kept blocks, so lane j of chunk c writes block 64 c + j at the row's
// position plus the kept blocks below it, and consecutive kept blocks go to
// consecutive addresses.  Blocks >= nb and positions at or past the head's
// capacity nb * nb are not written.
// ---------------------------------------------------------------------------
constexpr int kCompactRows = 16;   // rows per compaction unit

struct CompactArgs {
  const uint32_t* bits;   // [bh, nb, nw]
  const int32_t* count;   // [bh, nb]
  int32_t* row_ptr;       // [bh, nb + 1]
  int32_t* col_idx;       // [bh, nb * nb]
};

__device__ inline void compact_rows(const Geo& g, const CompactArgs& a, int64_t head, int r0,
                                    int n) {
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  const int nc = (nb + 63) >> 6;     // 64-block chunks per row
  const int lane = threadIdx.x & 63;
  const int32_t* cnt = a.count + head * nb;
  if (r0 + n > nb) n = nb - r0;
  // kept blocks of all rows before r0: four independent loads in flight per lane
  int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
  for (int i = lane; i < r0; i += 256) {
    s0 += cnt[i];
    if (i + 64 < r0) s1 += cnt[i + 64];
    if (i + 128 < r0) s2 += cnt[i + 128];
    if (i + 192 < r0) s3 += cnt[i + 192];
  }
  const int base = wave_sum_i((s0 + s1) + (s2 + s3));
  const int c = lane < n ? cnt[r0 + lane] : 0;
  int incl = c;                      // inclusive scan over the wavefront
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const int start = base + incl - c;
  int32_t* rp = a.row_ptr + head * (nb + 1);
  if (lane < n) rp[r0 + lane] = start;
  if (lane == n - 1 && r0 + n == nb) rp[nb] = base + incl;   // the head's last row
  int32_t* out = a.col_idx + head * (int64_t)nb * nb;
  const uint32_t cap = (uint32_t)nb * (uint32_t)nb;
  // every row's chunk words are loaded up front, so their latency is paid once
  const int w0 = 2 * lane, w1 = w0 + 1;
  uint32_t lo[kCompactRows], hi[kCompactRows];
#pragma unroll
  for (int ri = 0; ri < kCompactRows; ++ri) {
    const uint32_t* wrow = a.bits + (head * nb + r0 + ri) * (int64_t)nw;
    lo[ri] = ri < n && w0 < nw ? wrow[w0] : 0u;
    hi[ri] = ri < n && w1 < nw ? wrow[w1] : 0u;
  }
  // blocks past nb in the last chunk are dropped
  const int tail = nb - 64 * (nc - 1);
  const uint64_t last_mask = tail >= 64 ? ~0ull : ((1ull << tail) - 1ull);
  const uint64_t below = (1ull << lane) - 1ull;   // lanes below this one
#pragma unroll
  for (int ri = 0; ri < kCompactRows; ++ri) {
    if (ri < n) {                    // wavefront-uniform
      uint32_t pos = (uint32_t)__builtin_amdgcn_readlane(start, ri);
      for (int ch = 0; ch < nc; ++ch) {
        uint64_t b = (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)lo[ri], ch) |
                     ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi[ri], ch) << 32);
        if (ch == nc - 1) b &= last_mask;
        if (b == 0ull) continue;
        const uint32_t at = pos + (uint32_t)__popcll(b & below);
        if (((b >> lane) & 1ull) && at < cap) out[at] = 64 * ch + lane;
        pos += (uint32_t)__popcll(b);
      }
    }
  }
}

}  // namespace mask_detail
}  // namespace nabla
