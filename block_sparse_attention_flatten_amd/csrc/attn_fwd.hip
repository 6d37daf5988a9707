// Block-sparse attention forward over the kept N x N token blocks
// ("NABLA: Neighborhood Adaptive Block-Level Attention", gist.science,
// Methodology: expansion of the block mask back to token resolution;
// lsdiaocha.cn article, sec. 2 step 3: each kept reduced entry stands for a
// whole N x N block computed exactly).
//
// bf16 path with V in the Q/K layout (nabla_attn_fwd), gfx950 matrix cores.
// The pipelined kernel for V given as V^T tiles (attn_fwd_vt.hip) is the fast
// path; this one needs no V^T pass.  One workgroup serves TWO query blocks
// that see similar keys -- the same 8x8 patch in two consecutive frames (an
// odd last frame pairs horizontal neighbours) -- and walks the merged,
// ascending union of their kept lists: every K/V tile in the union is fetched
// once for both.  Four wavefronts: 0-1 own the first query block, 2-3 the
// second, 32 queries each.  For every block of the union:
//   * all 256 threads load the K and V tiles (64 x d bf16 each) into LDS; the
//     next tile of the union is prefetched into registers meanwhile;
//   * a wavefront whose query block does not keep this key block skips it;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so the 32 scores a lane
//     holds belong to ONE query: the online softmax needs one cross-lane
//     exchange (lane l <-> l^32) per block for the row max and none for the
//     row sum (each lane keeps a partial sum);
//   * P^T is converted to bf16 in registers and used directly as the B
//     operand of O^T += V^T P^T; the V^T operand comes from the row-major V
//     tile through ds_read_b64_tr_b16 transpose loads;
//   * the running max only moves when a block's max exceeds it by more than
//     2^8 in the exp2 domain (exact: O and the row sum share the reference).
// Pad keys (latent edge blocks) get -inf scores; pad queries are not written
// (blocked layout: written as zeros).
//
// fp32 path: one query block per workgroup on fp32 matrix cores, K/V tiles
// in LDS (below), used for float32 inputs.
#include "attn_common.hpp"

namespace nabla {

namespace {

template <int D>
struct AttnShape {
  // LDS row strides (elements).  K rows are read as 16-byte operand rows by 32
  // lanes: a stride of 4 (mod 32) banks spreads 8 consecutive rows over all
  // banks.  V rows are read by transpose loads, 4 rows x 32 bytes per 16-lane
  // group: a stride of 8 (mod 32) banks keeps those 4 rows disjoint.
  static constexpr int kStride = D + 8;
  static constexpr int kVStride = D + 16;
  static constexpr int kThreads = 256;
  static constexpr int kChunks = D / 8;           // 16-byte chunks per token row
  static constexpr int kRowsPerPass = kThreads / kChunks;
  static constexpr int kPasses = kN / kRowsPerPass;
  static constexpr int kSteps = D / 16;           // k-steps of S^T = K Q^T
  static constexpr int kDTiles = D / 32;          // 32-row tiles of O^T
};

// V is in the Q/K layout; its matrix-core operands come from transpose loads.
template <int D, typename OutT>
__global__ void __launch_bounds__(256, 2)
attn_fwd_bf16_kernel(const Geo g, const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const int32_t* __restrict__ row_ptr,
                     const int32_t* __restrict__ col_idx, float scale_log2,
                     OutT* __restrict__ O, float* __restrict__ lse) {
  using A = AttnShape<D>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[kN * A::kStride];
  __shared__ __attribute__((aligned(16))) __bf16 Vs[kN * A::kVStride];

  const int nb = g.nb;
  const int items = pair_items(g);
  int64_t head;
  int item;
  if (!xcd_item(blockIdx.x, items, (items + 7) >> 3, &head, &item)) return;
  int qa, qpair;
  pair_of(g, item, &qa, &qpair);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 1;         // 0: first query block of the pair, 1: second
  const int hl = lane >> 5;          // lane half
  const int jl = lane & 31;          // query column / operand row of this lane
  const int myq = grp == 0 ? qa : qpair;   // -1: this wavefront only helps load
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);

  // ---- this lane's query row as the B operand of S^T = K Q^T ----
  const int qs = 32 * (wave & 1) + jl;   // slot in the query block
  bool qvalid = false;
  int64_t qoff = 0;
  if (myq >= 0) {
    const BlockCoord qc = block_coord(g, myq);
    qvalid = (qs >> 3) < block_rows_valid(g, qc) && (qs & 7) < block_cols_valid(g, qc);
    qoff = hoff + block_base(g, myq, qc) + (qs >> 3) * row_step + (qs & 7) * D;
  }
  bf16x8 qop[A::kSteps];
#pragma unroll
  for (int s = 0; s < A::kSteps; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qvalid) raw = *(const u32x4*)(Q + qoff + 16 * s + 8 * hl);
    qop[s] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x16 oacc[A::kDTiles];
#pragma unroll
  for (int t = 0; t < A::kDTiles; ++t) oacc[t] = f32x16{};
  // running max (exp2 domain) of this lane's query; a finite start keeps a
  // block whose keys are all masked (scores -inf) at p = exp2(-inf) = 0
  float m_run = -1e30f;
  float l_run = 0.f;                 // partial row sum over the keys this lane holds

  const int32_t* rp = row_ptr + head * (nb + 1);
  const int32_t* cols = col_idx + head * (int64_t)nb * nb;
  KeptList la = kept_list(rp, cols, nb, qa);
  KeptList lb = kept_list(rp, cols, nb, qpair);

  // loader mapping: thread -> (chunk, first row); rows advance by kRowsPerPass
  const int ld_chunk = tid % A::kChunks;
  const int ld_row = tid / A::kChunks;
  u32x4 kreg[A::kPasses], vreg[A::kPasses];

  // Pad key rows (latent edge) load row 0 of the same block instead: any
  // finite data will do, since their scores are set to -inf and their P to 0.
  auto fetch = [&](int beta) {
    const BlockCoord bc = block_coord(g, beta);
    const int rv = block_rows_valid(g, bc);
    const int cv = block_cols_valid(g, bc);
    const __bf16* kb = K + hoff + block_base(g, beta, bc) + ld_chunk * 8;
    const __bf16* vb = V + hoff + block_base(g, beta, bc) + ld_chunk * 8;
#pragma unroll
    for (int p = 0; p < A::kPasses; ++p) {
      const int r = ld_row + p * A::kRowsPerPass;
      const bool ok = (r >> 3) < rv && (r & 7) < cv;
      const int off = ok ? (r >> 3) * row_step + (r & 7) * D : 0;
      kreg[p] = *(const u32x4*)(kb + off);
      vreg[p] = *(const u32x4*)(vb + off);
    }
  };

  int next = min(la.head, lb.head);          // next key block of the merged union
  if (next != INT_MAX) fetch(next);
  while (next != INT_MAX) {
    const int beta = next;
    const bool in_a = la.head == beta;
    const bool in_b = lb.head == beta;
    if (in_a) { ++la.i; la.settle(); }
    if (in_b) { ++lb.i; lb.settle(); }
    next = min(la.head, lb.head);
    __syncthreads();                 // every wavefront is done with the previous tile
#pragma unroll
    for (int p = 0; p < A::kPasses; ++p) {
      const int r = ld_row + p * A::kRowsPerPass;
      *(u32x4*)(Ks + r * A::kStride + ld_chunk * 8) = kreg[p];
      *(u32x4*)(Vs + r * A::kVStride + ld_chunk * 8) = vreg[p];
    }
    __syncthreads();
    if (next != INT_MAX) fetch(next);
    if (!(grp == 0 ? in_a : in_b)) continue;   // wavefront-uniform: not a kept block of ours

    // ---- S^T (64 keys x 32 queries) ----
    // Operand reads are issued ahead of the matrix instructions that use them
    // (all of key tile 0, then one of key tile 1 per instruction of tile 0),
    // so LDS latency overlaps matrix work instead of stalling every
    // instruction; the scheduling-group barriers at the end pin that order.
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    bf16x8 ka[A::kSteps], kb2[A::kSteps];
#pragma unroll
    for (int s = 0; s < A::kSteps; ++s)
      ka[s] = *(const bf16x8*)(Ks + jl * A::kStride + 16 * s + 8 * hl);
#pragma unroll
    for (int s = 0; s < A::kSteps; ++s) {
      sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qop[s], sacc[0], 0, 0, 0);
      kb2[s] = *(const bf16x8*)(Ks + (32 + jl) * A::kStride + 16 * s + 8 * hl);
    }
#pragma unroll
    for (int s = 0; s < A::kSteps; ++s)
      sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb2[s], qop[s], sacc[1], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, A::kSteps, 0);
#pragma unroll
    for (int s = 0; s < A::kSteps; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, A::kSteps, 0);
    // element r of sacc[kt] is key 32kt + 8(r/4) + 4hl + (r%4) of this lane's query
    const BlockCoord bc = block_coord(g, beta);
    const int rv = block_rows_valid(g, bc);
    const int cv = block_cols_valid(g, bc);
    if (rv < kP || cv < kP) {        // latent-edge block: pad keys get -inf
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (!((key >> 3) < rv && (key & 7) < cv)) sacc[kt][r] = -INFINITY;
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale_log2;
    // move the reference only when needed (wavefront-uniform decision)
    const bool grow = mx > m_run + 8.0f;
    if (__any(grow)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first block
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < A::kDTiles; ++t) oacc[t] *= alpha;
      m_run = m_new;
    }
    // P^T in bf16 (v_exp_f32 directly: its inputs are <= 8, and results below
    // the fp32 normal range flush to 0, which only drops weights < 2^-126);
    // the row sum adds the ROUNDED values (bf16 pairs summed in fp32 by
    // v_dot2_f32_bf16) so that O / l is an exact convex combination of V
    // under the weights the matrix cores actually used
    bf16x8 pop[2][2];
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = __builtin_fmaf(sacc[kt][8 * h + e], scale_log2, -m_run);
          const float x1 = __builtin_fmaf(sacc[kt][8 * h + e + 1], scale_log2, -m_run);
          const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(x0),
                             (__bf16)__builtin_amdgcn_exp2f(x1)};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
          pop[kt][h][e] = pr[0];
          pop[kt][h][e + 1] = pr[1];
        }
      }
    }
    // ---- O^T (d x 32 queries) += V^T P^T ----
    {
      // A operand (V^T rows d = 32dt + lane%32, keys k0..k0+3, k0+8..k0+11
      // with k0 = 32kt + 16h + 4hl) straight from the row-major V tile with
      // two transpose loads: in each 16-lane group, lane i receives element
      // i%4 of the 4-element rows addressed by lanes 4e + i/4 (e = 0..3), so
      // lane s of the group addresses key k0 + s/4 (+8), columns
      // d0 + 4(s%4) .. +3.
      const __bf16* vsrc = Vs + ((lane & 15) >> 2) * A::kVStride + (lane & 16) + 4 * (lane & 3);
#pragma unroll
      for (int dt = 0; dt < A::kDTiles; ++dt) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int k0 = 32 * kt + 16 * h + 4 * hl;
            const __bf16* src = vsrc + k0 * A::kVStride + 32 * dt;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(src));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) bf16x4*)(src + 8 * A::kVStride));
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop[kt][h], oacc[dt], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- normalise and write this lane's query row ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (lse != nullptr && myq >= 0 && hl == 0)   // ln sum exp(s * scale) = (m + log2 l) ln 2
    lse[(head * nb + myq) * kN + qs] =
        qvalid && l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (myq >= 0 && (qvalid || g.layout == 1)) {
    OutT* orow = O + qoff;
    const float sc = qvalid ? inv : 0.f;
#pragma unroll
    for (int dt = 0; dt < A::kDTiles; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        store4<OutT>(orow + 32 * dt + 8 * gq + 4 * hl, oacc[dt][4 * gq] * sc,
                     oacc[dt][4 * gq + 1] * sc, oacc[dt][4 * gq + 2] * sc,
                     oacc[dt][4 * gq + 3] * sc);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// float32 path on fp32 matrix cores (v_mfma_f32_16x16x4f32).  One workgroup of
// four wavefronts per query block walks its kept list; wavefront w owns
// queries 16w .. 16w + 15.  The K and V tiles (64 x d float32) are staged in
// LDS with rows padded by 16 bytes, so the 16 rows a read instruction touches
// fall on distinct banks.
//   * S^T = K Q^T: lane l supplies key row 16 kt + l % 16 and query l % 16;
//     the contraction index is permuted the same way for both operands
//     (step s, lane group r = l / 16 supplies element r d/4 + s), so each
//     lane's operands are contiguous.  The result gives lane l the scores of
//     query l % 16 against keys 16 kt + 4 (l / 16) + i, i < 4.
//   * O^T += V^T P^T: with keys ordered the same way inside each 4-key step,
//     the B operand is the lane's own score slot and the A operand one float
//     of the V tile, so P never leaves the registers.
//   * Online softmax in the exp2 domain in float32 (no rounding of P); the
//     row max is taken over the four lanes that share a query.
// Pad keys get -inf scores; pad queries are not written (blocked layout:
// zeros).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
attn_fwd_f32_kernel(const Geo g, const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, const int32_t* __restrict__ row_ptr,
                    const int32_t* __restrict__ col_idx, float scale_log2, float* __restrict__ O,
                    float* __restrict__ lse) {
  constexpr int kStride = D + 4;           // LDS row stride (floats)
  constexpr int kQ = D / 4;                // contraction steps per 16 x 16 score tile
  constexpr int kDT = D / 16;              // 16-channel tiles of O^T
  __shared__ __attribute__((aligned(16))) float Kt[kN * kStride];
  __shared__ __attribute__((aligned(16))) float Vt[kN * kStride];
  const int nb = g.nb;
  const int64_t head = blockIdx.x / nb;
  const int qb = (int)(blockIdx.x - head * nb);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, r = lane >> 4;
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);
  const BlockCoord qc = block_coord(g, qb);
  const int qs = 16 * wave + n;            // this lane's query slot in the block
  const bool qvalid = (qs >> 3) < block_rows_valid(g, qc) && (qs & 7) < block_cols_valid(g, qc);
  const int64_t qoff = hoff + block_base(g, qb, qc) + (qs >> 3) * row_step + (qs & 7) * D;

  float qop[kQ];                           // Q[qs][r d/4 + s]
#pragma unroll
  for (int c = 0; c < kQ; c += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (qvalid) x = *(const f32x4*)(Q + qoff + r * kQ + c);
    qop[c] = x[0]; qop[c + 1] = x[1]; qop[c + 2] = x[2]; qop[c + 3] = x[3];
  }
  f32x4 oacc[kDT];                         // O[qs][16 dt + 4 r + i]
#pragma unroll
  for (int t = 0; t < kDT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;    // exp2 domain; l_run: this lane's keys only

  const int32_t* rp = row_ptr + head * (nb + 1);
  const int32_t* cols = col_idx + head * (int64_t)nb * nb;
  const int begin = rp[qb];
  int end = rp[qb + 1];
  if (begin < 0 || end < begin || end > nb * nb) end = begin;   // malformed row: no keys
  for (int idx = begin; idx < end; ++idx) {
    const int beta = cols[idx];
    if ((unsigned)beta >= (unsigned)nb) continue;               // uniform across the block
    const BlockCoord bc = block_coord(g, beta);
    const int rv = block_rows_valid(g, bc), cv = block_cols_valid(g, bc);
    const int64_t base = hoff + block_base(g, beta, bc);
    __syncthreads();
    for (int i = threadIdx.x; i < kN * D / 4; i += 256) {
      const int row = i / (D / 4), c4 = i % (D / 4);
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if ((row >> 3) < rv && (row & 7) < cv) {
        const int64_t off = base + (row >> 3) * row_step + (row & 7) * D + 4 * c4;
        kv = *(const f32x4*)(K + off);
        vv = *(const f32x4*)(V + off);
      }
      *(f32x4*)(Kt + row * kStride + 4 * c4) = kv;
      *(f32x4*)(Vt + row * kStride + 4 * c4) = vv;
    }
    __syncthreads();
    // scores of this lane's query against keys 16 kt + 4 r + i
    f32x4 sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const float* krow = Kt + (16 * kt + n) * kStride + r * kQ;
#pragma unroll
      for (int c = 0; c < kQ; c += 4) {
        const f32x4 a = *(const f32x4*)(krow + c);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], qop[c + j], acc, 0, 0, 0);
      }
      sc[kt] = acc;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 16 * kt + 4 * r + i;
        const bool ok = (key >> 3) < rv && (key & 7) < cv;
        sc[kt][i] = ok ? sc[kt][i] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, sc[kt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: every kept block has a valid key
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first block
    m_run = m_new;
    l_run *= corr;
#pragma unroll
    for (int t = 0; t < kDT; ++t) oacc[t] *= corr;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[kt][i] - m_new);   // pad keys: 0
        l_run += p;
        const float* vrow = Vt + (16 * kt + 4 * r + i) * kStride + n;
#pragma unroll
        for (int t = 0; t < kDT; ++t)
          oacc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * t], p, oacc[t], 0, 0, 0);
      }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (lse != nullptr && r == 0)            // ln sum exp(s * scale) = (m + log2 l) ln 2
    lse[(head * nb + qb) * kN + qs] =
        qvalid && l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (qvalid || g.layout == 1) {
    // oacc[t][i] = O^T[16 t + 4 r + i][n]; a store per lane group of 4 channels
    const float inv = qvalid && l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int t = 0; t < kDT; ++t)
      *(f32x4*)(O + qoff + 16 * t + 4 * r) = oacc[t] * inv;
  }
}

template <int D, typename OutT>
void launch_bf16(const Geo& g, const void* q, const void* k, const void* v,
                 const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                 float* lse, hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;   // softmax in base 2
  const int64_t chunk = (pair_items(g) + 7) / 8;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, OutT>), dim3((unsigned)(8 * chunk * g.bh)),
                     dim3(AttnShape<D>::kThreads), 0, s, g, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, row_ptr, col_idx, sl2, (OutT*)o, lse);
}

void launch_bf16_any(const Geo& g, bool out_bf16, const void* q, const void* k, const void* v,
                     const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                     float* lse, hipStream_t s) {
  if (g.d == 64) {
    out_bf16 ? launch_bf16<64, __bf16>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s)
             : launch_bf16<64, float>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s);
  } else {
    out_bf16 ? launch_bf16<128, __bf16>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s)
             : launch_bf16<128, float>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s);
  }
}

template <int D>
void launch_f32(const Geo& g, const void* q, const void* k, const void* v,
                const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                float* lse, hipStream_t s) {
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)(g.bh * g.nb)), dim3(256), 0, s, g,
                     (const float*)q, (const float*)k, (const float*)v, row_ptr, col_idx,
                     scale * 1.4426950408889634f, (float*)o, lse);
}

}  // namespace

hipError_t launch_attn_fwd(const Geo& g, bool bf16, bool out_bf16, const void* q, const void* k,
                           const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                           float scale, void* o, float* lse, hipStream_t s) {
  if (bf16) {
    launch_bf16_any(g, out_bf16, q, k, v, row_ptr, col_idx, scale, o, lse, s);
  } else {
    g.d == 64 ? launch_f32<64>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s)
              : launch_f32<128>(g, q, k, v, row_ptr, col_idx, scale, o, lse, s);
  }
  return hipGetLastError();
}


}  // namespace nabla
