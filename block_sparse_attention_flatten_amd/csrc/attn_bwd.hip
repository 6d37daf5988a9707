// Gradients of the block-sparse attention with the kept-block mask held fixed
// (training with NABLA: "NABLA: Neighborhood Adaptive Block-Level Attention",
// gist.science, core contributions -- pre-training / fine-tuning speed-up --
// and experimental results 2, pre-training of a 2B DiT; lsdiaocha.cn article,
// sec. 3).  The mask is a threshold on pooled scores, so only the exact
// attention over the kept N x N blocks is differentiated:
//   p = softmax(s), s = q k^T * scale;  dv = p^T do;  dp = do v^T;
//   ds = p (dp - D), D = rowsum(do * o);  dq = ds k * scale;  dk = ds^T q * scale.
// p is recomputed from the forward's log-sum-exp, so no N x N matrix is kept.
//
// Three calls:
//   * mask transpose: key block c's list of the query blocks that keep it
//     (bit r of transposed row c = bit c of row r), compacted by nabla_compact;
//   * dQ: one workgroup per PAIR of query blocks walking the union of their
//     kept lists (as the forward does), K and V tiles by direct-to-LDS loads
//     into double buffers; per kept block S^T = K Q^T and
//     dP^T = V dO^T on the matrix cores, dS^T in registers, and
//     dQ^T += K^T dS^T with K^T operands from transpose loads of the K tile.
//     It also writes D = rowsum(dO * O) for the second call;
//   * dK / dV: one workgroup per key block walking its query-block list, Q
//     and dO tiles (and the block's lse and D) by direct-to-LDS loads.
//     Wavefronts 0-1 compute S = Q K^T and P and accumulate dV^T += dO^T P;
//     they hand P to wavefronts 2-3, which compute dP = dO V^T and
//     accumulate dK^T += Q^T dS.  32 keys per wavefront, so each lane owns
//     one key and every accumulation stays in registers; S is computed once.
// float32 inputs use plain per-thread kernels of the same structure.
#include <type_traits>

#include "attn_common.hpp"

namespace nabla {

namespace {

// ---------------------------------------------------------------------------
// transposed mask
// ---------------------------------------------------------------------------
// One wavefront per transposed row c (grid: nb x bh): 64 source rows per step,
// the wanted bit of each gathered by a ballot.
__global__ void __launch_bounds__(64)
mask_transpose_kernel(const Geo g, const uint32_t* __restrict__ bits,
                      uint32_t* __restrict__ bits_t, int32_t* __restrict__ count_t) {
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  const int c = blockIdx.x;
  const int64_t head = blockIdx.y;
  const int lane = threadIdx.x;
  const uint32_t* src = bits + head * (int64_t)nb * nw + (c >> 5);
  uint32_t* dst = bits_t + (head * nb + c) * (int64_t)nw;
  int cnt = 0;
  for (int r0 = 0; r0 < nb; r0 += 64) {
    const int r = r0 + lane;
    const bool b = r < nb && ((src[(int64_t)r * nw] >> (c & 31)) & 1u);
    const uint64_t m = __ballot(b);
    const int w = r0 >> 5;
    if (lane == 0) dst[w] = (uint32_t)m;
    if (lane == 1 && w + 1 < nw) dst[w + 1] = (uint32_t)(m >> 32);
    cnt += __popcll(m);
  }
  if (lane == 0) count_t[head * nb + c] = cnt;
}

// ---------------------------------------------------------------------------
// bf16 kernels
// ---------------------------------------------------------------------------
template <int D>
struct BwdShape {
  static constexpr int kSteps = D / 16;           // k-steps over d
  static constexpr int kDTiles = D / 32;          // 32-row tiles of a d x 32 accumulator
};

constexpr float kLog2e = 1.4426950408889634f;

// A lane's token row as matrix-core operand chunks: chunk s holds elements
// 16 s + 8 hl .. + 7 (zero when the row is not valid).
template <int D>
__device__ inline void row_operand(const __bf16* X, int64_t off, bool valid, int hl,
                                   bf16x8 (&op)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (valid) raw = *(const u32x4*)(X + off + 16 * s + 8 * hl);
    op[s] = __builtin_bit_cast(bf16x8, raw);
  }
}

// Accumulator element r of a 32 x 32 tile sits in row 8 (r / 4) + 4 hl + r % 4
// of this lane's column; as a B operand over those 32 rows, k-step h takes
// elements 8 h .. 8 h + 7 (element e of operand h is accumulator element
// 8 h + e).

// store a lane's d-vector held as accumulator columns: element r of tile dt is
// component 32 dt + 8 (r / 4) + 4 hl + r % 4
template <int D>
__device__ inline void store_row(__bf16* dst, const f32x16 (&acc)[D / 32], float mul, int hl) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
      store4<__bf16>(dst + 32 * dt + 8 * gq + 4 * hl, acc[dt][4 * gq] * mul,
                     acc[dt][4 * gq + 1] * mul, acc[dt][4 * gq + 2] * mul,
                     acc[dt][4 * gq + 3] * mul);
}

// ---- swizzled tiles filled by direct-to-LDS loads ----
// A 64 x D bf16 tile whose 16-byte chunks are permuted within each row so that
// the 16-byte row reads of 16 consecutive rows (one logical chunk) hit
// distinct banks: 256-byte rows (D = 128) use chunk ^ g(r) plus 128 bytes of
// padding after every 8 rows; 128-byte rows (D = 64) use chunk ^
// ((r & 7) ^ ((r >> 3) & 1)).  g(r) = ((r & 3) << 1) | ((r >> 2) & 1) permutes
// each 8-row group (row reads stay conflict-free) and also gives 4
// consecutive rows distinct values of g >> 1, so the transposing reads, where
// 16 lanes take chunks 2m and 2m + 1 of 4 consecutive rows, hit 8 distinct
// bank groups; with r & 7 rows 2k and 2k + 1 collided, and the bank-conflict
// counter read about half of the LDS-active cycles in both kernels.  The
// tile is filled in 1-KB direct loads:
// lane l of a load writes bytes 16 l .. 16 l + 15 of it and reads the global
// chunk that belongs there.
template <int D>
struct SwTile {
  static constexpr bool kWide = D == 128;
  static constexpr int kGroupBytes = kWide ? 8 * 256 + 128 : 8 * 128;   // 8 rows
  static constexpr int kBytes = 8 * kGroupBytes;
  static constexpr int kOps = kN * D * 2 / 1024;          // 1-KB loads per tile
  __device__ static int swz(int r) {
    return kWide ? (((r & 3) << 1) | ((r >> 2) & 1)) : ((r & 7) ^ ((r >> 3) & 1));
  }
  // byte offset of logical chunk c of row r
  __device__ static int addr(int r, int c) {
    return (r >> 3) * kGroupBytes + (r & 7) * (2 * D) + ((c ^ swz(r)) << 4);
  }
  // load o: the row and logical chunk this lane moves, and the load's LDS offset
  __device__ static void op_rc(int o, int lane, int* r, int* c) {
    if (kWide) {
      *r = 4 * o + (lane >> 4);
      *c = (lane & 15) ^ swz(*r);
    } else {
      *r = 8 * o + (lane >> 3);
      *c = (lane & 7) ^ swz(*r);
    }
  }
  __device__ static int op_dst(int o) {
    return kWide ? (o >> 1) * kGroupBytes + (o & 1) * 1024 : o * 1024;
  }
};

// Wavefront `wave`'s share (kOps / 4 loads) of the tile of block blk of the
// tensor behind rs into the tile at LDS byte address dst.  Pad rows of a
// latent-edge block load row 0 of the block.
template <int D>
__device__ inline void dma_tile(const Geo& g, __amdgpu_buffer_rsrc_t rs, int row_step, int blk,
                                int wave, int lane, char* dst) {
  using T = SwTile<D>;
  const BlockCoord bc = block_coord(g, blk);
  const int rv = block_rows_valid(g, bc), cv = block_cols_valid(g, bc);
  const uint32_t sb = 2u * (uint32_t)block_base(g, blk, bc);
#pragma unroll
  for (int i = 0; i < T::kOps / 4; ++i) {
    const int o = wave * (T::kOps / 4) + i;
    int r, c;
    T::op_rc(o, lane, &r, &c);
    const bool ok = (r >> 3) < rv && (r & 7) < cv;
    // a head holds at most 2^26 bytes, so 2^31 is out of range even with sb added
    const uint32_t voff = ok ? 2u * (uint32_t)((r >> 3) * row_step + (r & 7) * D + c * 8)
                             : 0x80000000u;
    dma16(rs, voff, sb, dst + T::op_dst(o));
  }
}

// A operand of a 32 x 32 x 16 product over d: tile row `row` of the swizzled
// tile at LDS address tb, k-step st (elements 16 st + 8 hl .. + 7), by one
// 16-byte read.
template <int D>
__device__ inline bf16x8 sw_row_read(int tb, int row, int st, int hl) {
  return lds_read16(tb + SwTile<D>::addr(row, 2 * st + hl));
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16) at base + off.  Through
// the restrict parameter the inlined read carries an alias scope, and the
// compiler's wait insertion then stops treating it as a possible reader of
// every direct-to-LDS load still in flight: without it, each step's first
// transposing read waited (vmcnt(0)) for the NEXT step's tile loads, so they
// had only the first half of a step to land.  The kernels order their reads
// after the loads they read by their own waits and barriers.
__device__ inline bf16x4 lds_read_tr8(lds_char* __restrict__ base, int off) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
}

// A operand of acc[dt] += X^T[32 dt + lane % 32][rows] * B over the 16 tile
// rows row0 + 16 h .. + 15 of the swizzled tile at LDS address tb (the
// product over tile rows, X^T from transpose loads).  In each 16-lane group,
// lane i receives element i % 4 of the 4-element rows addressed by lanes
// 4e + i / 4, so the lane supplying rows k0 + s / 4 and k0 + 8 + s / 4
// (k0 = row0 + 16 h + 4 hl), columns 32 dt + (lane & 16) + 4 (s % 4), yields
// exactly the k order of a B operand built from a 32 x 32 accumulator.
template <int D>
__device__ inline bf16x8 sw_tr_read(int tb, int row0, int h, int dt, int lane) {
  const int col = 32 * dt + (lane & 16) + 4 * (lane & 3);
  const int r = row0 + 16 * h + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int c = (col & 7) * 2;
  lds_char* const base = (lds_char*)(uintptr_t)tb;
  const bf16x4 lo = lds_read_tr8(base, SwTile<D>::addr(r, col >> 3) + c);
  const bf16x4 hi = lds_read_tr8(base, SwTile<D>::addr(r + 8, col >> 3) + c);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// N matrix instructions in a fixed order, the A operand of slot i read
// kAhead slots earlier so that LDS latency overlaps the matrix work:
// read(j) returns slot j's A operand, mma(i, a) issues slot i's instruction,
// work(i) is the vector work placed beside it.  The scheduling barrier keeps
// each slot's content together.
template <int N, typename Read, typename Mma, typename Work>
__device__ inline void run_slots(Read read, Mma mma, Work work) {
  constexpr int kAhead = N < 3 ? N : 3;
  bf16x8 a[N];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) a[j] = read(j);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    mma(i, a[i]);
    work(i);
    if (i + kAhead < N) a[i + kAhead] = read(i + kAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
}

__device__ inline f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- dQ (and D) ----
// K and V tiles move by direct-to-LDS loads into two buffers each: step s
// loads the next union block's tiles while computing on the current ones,
// with one barrier per step.
template <int D>
__global__ void __launch_bounds__(256, 2)
attn_bwd_dq_kernel(const Geo g, const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ O,
                   const __bf16* __restrict__ dO, const float* __restrict__ lse,
                   const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                   float scale_log2, float scale, __bf16* __restrict__ dQ,
                   float* __restrict__ delta) {
  using A = BwdShape<D>;
  using T = SwTile<D>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];   // K[2], V[2] tiles

  const int nb = g.nb;
  const int items = pair_items(g);
  int64_t head;
  int item;
  if (!xcd_item(blockIdx.x, items, (items + 7) >> 3, &head, &item)) return;
  int qa, qpair;
  pair_of(g, item, &qa, &qpair);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 1;
  const int hl = lane >> 5;
  const int jl = lane & 31;
  const int myq = grp == 0 ? qa : qpair;
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K + hoff, 2u * (uint32_t)g.head_elems);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(V + hoff, 2u * (uint32_t)g.head_elems);
  const int lds0 = (int)(uintptr_t)(lds_char*)smem;

  // this lane's query row: Q and dO as B operands, D = rowsum(dO * O)
  const int qs = 32 * (wave & 1) + jl;
  bool qvalid = false;
  int64_t qoff = 0;
  if (myq >= 0) {
    const BlockCoord qc = block_coord(g, myq);
    qvalid = (qs >> 3) < block_rows_valid(g, qc) && (qs & 7) < block_cols_valid(g, qc);
    qoff = hoff + block_base(g, myq, qc) + (qs >> 3) * row_step + (qs & 7) * D;
  }
  bf16x8 qop[A::kSteps], doop[A::kSteps];
  row_operand<D>(Q, qoff, qvalid, hl, qop);
  row_operand<D>(dO, qoff, qvalid, hl, doop);
  float dpart = 0.f;
#pragma unroll
  for (int s = 0; s < A::kSteps; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qvalid) raw = *(const u32x4*)(O + qoff + 16 * s + 8 * hl);
    const bf16x8 o8 = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = fmaf((float)doop[s][e], (float)o8[e], dpart);
  }
  const float Dq = dpart + __shfl_xor(dpart, 32);
  const int64_t slot = myq >= 0 ? (head * nb + myq) * kN + qs : 0;
  if (myq >= 0 && hl == 0) delta[slot] = qvalid ? Dq : 0.f;
  // p = exp2(s * scale_log2 - lse2); pad queries get lse2 = +inf, i.e. p = 0
  float lse2 = INFINITY;
  if (myq >= 0 && qvalid) {
    const float l = lse[slot];
    if (l > -INFINITY) lse2 = l * kLog2e;
  }

  f32x16 dqacc[A::kDTiles];
#pragma unroll
  for (int t = 0; t < A::kDTiles; ++t) dqacc[t] = f32x16{};

  const int32_t* rp = row_ptr + head * (nb + 1);
  const int32_t* cols = col_idx + head * (int64_t)nb * nb;
  KeptList la = kept_list(rp, cols, nb, qa);
  KeptList lb = kept_list(rp, cols, nb, qpair);
  auto load = [&](int blk, int buf) {
    dma_tile<D>(g, krs, row_step, blk, wave, lane, smem + buf * T::kBytes);
    dma_tile<D>(g, vrs, row_step, blk, wave, lane, smem + (2 + buf) * T::kBytes);
  };
  int cur = min(la.head, lb.head);           // current block of the merged union
  if (cur != INT_MAX) load(cur, 0);
  for (int s = 0; cur != INT_MAX; ++s) {
    const bool in_a = la.head == cur;
    const bool in_b = lb.head == cur;
    if (in_a) { ++la.i; la.settle(); }
    if (in_b) { ++lb.i; lb.settle(); }
    const int next = min(la.head, lb.head);
    wait_vmcnt0();                   // this wavefront's loads of cur have landed
    __syncthreads();                 // ... everyone's, and everyone is done with the other buffer
    if (next != INT_MAX) load(next, (s + 1) & 1);
    if (grp == 0 ? in_a : in_b) {    // wavefront-uniform: a kept block of ours
      const int kb = lds0 + (s & 1) * T::kBytes;
      const int vb = lds0 + (2 + (s & 1)) * T::kBytes;
      // One run of 4 kSteps + 4 kDTiles matrix instructions, for keys
      // 32 kt .. 32 kt + 31 (kt = 0, 1) of the block and this lane's query:
      //   S^T(0) = K Q^T, dP^T(0) = V dO^T, S^T(1), dP^T(1)   (tile rows),
      //   dQ^T += K^T dS^T for kt = 0, then 1                 (transpose loads),
      // with the vector work of one stage beside the next one's products:
      // p = exp2(S scale log2(e) - lse log2(e)) of half kt beside dP^T(kt),
      // dS^T(0) = P (dP - D) beside S^T(1), dS^T(1) beside the kt = 0 dQ
      // products.
      constexpr int kR = A::kSteps;                  // slots per row product
      constexpr int kQ = 2 * A::kDTiles;             // dQ slots per half
      f32x16 sacc[2], dpacc[2];
      bf16x8 b[2][2];                                // dS^T as B operands
      // Pad keys (zero rows of the K and V tiles) need no mask: S = dP = 0
      // there, and K^T's zero rows drop their dS from dQ.  Their p =
      // exp2(-lse log2(e)) is clamped to 2^64 so that dS stays finite (real
      // keys have S scale log2(e) - lse log2(e) <= 0, untouched by the clamp).
      auto exps = [&](int kt, int r) {
        sacc[kt][r] =
            __builtin_amdgcn_exp2f(fminf(fmaf(sacc[kt][r], scale_log2, -lse2), 64.0f));
      };
      auto ds = [&](int kt, int r) {
        b[kt][r >> 3][r & 7] = (__bf16)(sacc[kt][r] * (dpacc[kt][r] - Dq));
      };
      run_slots<4 * kR + 2 * kQ>(
          [&](int j) {
            if (j < 4 * kR) {
              const int part = j / kR;               // S(0), dP(0), S(1), dP(1)
              return sw_row_read<D>((part & 1) ? vb : kb, 32 * (part >> 1) + jl, j % kR, hl);
            }
            const int jj = j - 4 * kR;
            return sw_tr_read<D>(kb, 32 * (jj / kQ), (jj / A::kDTiles) & 1, jj % A::kDTiles,
                                 lane);
          },
          [&](int i, bf16x8 a) {
            if (i < 4 * kR) {
              const int part = i / kR, st = i % kR, kt = part >> 1;
              if (part & 1)
                dpacc[kt] = mfma_bf16(a, doop[st], st == 0 ? f32x16{} : dpacc[kt]);
              else
                sacc[kt] = mfma_bf16(a, qop[st], st == 0 ? f32x16{} : sacc[kt]);
            } else {
              const int jj = i - 4 * kR;
              const int dt = jj % A::kDTiles;
              dqacc[dt] = mfma_bf16(a, b[jj / kQ][(jj / A::kDTiles) & 1], dqacc[dt]);
            }
          },
          [&](int i) {
            constexpr int kPer = 16 / kR;            // elements per row-product slot
            if (i < 4 * kR) {
              const int part = i / kR, st = i % kR;
              if (part == 1 || part == 3) {          // beside dP(kt): exponentials of half kt
#pragma unroll
                for (int e = 0; e < kPer; ++e) exps(part >> 1, st * kPer + e);
              } else if (part == 2) {                // beside S(1): dS(0)
#pragma unroll
                for (int e = 0; e < kPer; ++e) ds(0, st * kPer + e);
              }
            } else if (i - 4 * kR < kQ) {            // beside the first dQ half: dS(1)
              constexpr int kPerQ = 16 / kQ;
#pragma unroll
              for (int e = 0; e < kPerQ; ++e) ds(1, (i - 4 * kR) * kPerQ + e);
            }
          });
    }
    cur = next;
  }

  if (myq >= 0 && (qvalid || g.layout == 1))
    store_row<D>(dQ + qoff, dqacc, qvalid ? scale : 0.f, hl);
}

// ---- dK and dV ----
// Q and dO tiles move by direct-to-LDS loads into two buffers each, with the
// 64 log-sum-exps and D values of the query block beside them.  Two barriers
// per step: after the first, the dV side computes S and P and hands P (bf16)
// to the dK side through LDS while the dK side computes dP; after the second,
// the dV side accumulates dV^T += dO^T P and the dK side dK^T += Q^T dS with
// dS = P (dP - D).  Every wavefront issues 4 x 8 matrix instructions per step,
// with its LDS operand reads issued several instructions ahead.
template <int D>
__global__ void __launch_bounds__(256, 2)
attn_bwd_dkdv_kernel(const Geo g, const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ lse, const float* __restrict__ delta,
                     const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
                     float scale_log2, float scale, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV) {
  using A = BwdShape<D>;
  using T = SwTile<D>;
  // Q[2], dO[2] tiles, lse[2][64] and D[2][64] (float), then P (8 KB)
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int nb = g.nb;
  int64_t head;
  int beta;
  if (!xcd_item(blockIdx.x, nb, (nb + 7) >> 3, &head, &beta)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dk_side = (wave >> 1) != 0;   // wavefronts 0-1: dV, 2-3: dK
  const int hl = lane >> 5;
  const int jl = lane & 31;
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(Q + hoff, 2u * (uint32_t)g.head_elems);
  const __amdgpu_buffer_rsrc_t grs = buffer_rsrc(dO + hoff, 2u * (uint32_t)g.head_elems);
  const uint32_t vec_bytes = 4u * (uint32_t)(nb * kN);
  const __amdgpu_buffer_rsrc_t lrs = buffer_rsrc(lse + head * nb * kN, vec_bytes);
  const __amdgpu_buffer_rsrc_t drs = buffer_rsrc(delta + head * nb * kN, vec_bytes);
  const int lds0 = (int)(uintptr_t)(lds_char*)smem;
  char* const vec = smem + 4 * T::kBytes;                 // lse[2][64], D[2][64]
  // P of a step, bf16, in the B-operand order of the dV side: [key half][qt][h]
  // blocks of 1 KB, 16 bytes per lane; the dK lane with the same key reads it
  char* const pbuf = vec + 1024;
  const int pslot = (wave & 1) * 4096 + lane * 16;

  // this lane's key row: K on the dV side (S = Q K^T), V on the dK side
  // (dP = dO V^T), as B operands
  const int ks = 32 * (wave & 1) + jl;
  const BlockCoord kc = block_coord(g, beta);
  const bool kvalid = (ks >> 3) < block_rows_valid(g, kc) && (ks & 7) < block_cols_valid(g, kc);
  const int64_t koff = hoff + block_base(g, beta, kc) + (ks >> 3) * row_step + (ks & 7) * D;
  bf16x8 rop[A::kSteps];
  row_operand<D>(dk_side ? V : K, koff, kvalid, hl, rop);
  f32x16 acc[A::kDTiles];
#pragma unroll
  for (int t = 0; t < A::kDTiles; ++t) acc[t] = f32x16{};

  KeptList lq = kept_list(col_ptr + head * (nb + 1), row_idx + head * (int64_t)nb * nb, nb, beta);
  // wavefront 0 moves the lse and D vectors first, so that it can wait for
  // them alone (vmcnt counts its loads in order) and rewrite the lse in place
  // as exp2-domain offsets: lse * log2(e), +inf for pad queries (weight 0)
  constexpr int kTileOps = 2 * (T::kOps / 4);            // per wavefront and step
  auto load = [&](int alpha, int buf) {
    if (wave == 0) {                 // 64 x 4 bytes each: lane l writes float l
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void*)(vec + buf * 256), 4, 4u * lane,
                                               4u * (uint32_t)(alpha * kN), 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void*)(vec + 512 + buf * 256), 4,
                                               4u * lane, 4u * (uint32_t)(alpha * kN), 0, 0);
#endif
    }
    dma_tile<D>(g, qrs, row_step, alpha, wave, lane, smem + buf * T::kBytes);
    dma_tile<D>(g, grs, row_step, alpha, wave, lane, smem + (2 + buf) * T::kBytes);
  };
  auto lse_to_exp2 = [&](int buf) {  // wavefront 0, after its vector loads landed
    float* l = (float*)(vec + buf * 256);
    const float v = l[lane];
    l[lane] = v > -INFINITY ? v * kLog2e : INFINITY;
  };

  // Barrier for LDS data only: waits for this wavefront's LDS accesses, not
  // for its direct-to-LDS loads of the next step (which a fence, and hence
  // __syncthreads, would also wait for).  The clobber keeps the compiler from
  // moving memory accesses across it.
  auto lds_barrier = [] { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // 2 kSteps slots: the 32 x 32 products over d for queries 32 qt .. +31,
  // qt = 0 then 1 (accumulation chains issue back to back), A operands from
  // the rows of the tile at tb, B = this lane's key row
  auto rows_slots = [&](int tb, f32x16 (&out)[2], auto work) {
    run_slots<2 * A::kSteps>(
        [&](int j) { return sw_row_read<D>(tb, 32 * (j / A::kSteps) + jl, j % A::kSteps, hl); },
        [&](int i, bf16x8 a) {
          const int qt = i / A::kSteps, st = i % A::kSteps;
          out[qt] = mfma_bf16(a, rop[st], st == 0 ? f32x16{} : out[qt]);
        },
        work);
  };
  // 4 kDTiles slots: acc[dt] += X^T(d rows 32 dt.., queries 32 qt + 16 h ..) b[qt][h]
  auto cols_slots = [&](int tb, const bf16x8 (&b)[2][2], auto work) {
    run_slots<4 * A::kDTiles>(
        [&](int j) {
          return sw_tr_read<D>(tb, 32 * (j / (2 * A::kDTiles)), (j / A::kDTiles) & 1,
                               j % A::kDTiles, lane);
        },
        [&](int i, bf16x8 a) {
          const int qt = i / (2 * A::kDTiles), h = (i / A::kDTiles) & 1, dt = i % A::kDTiles;
          acc[dt] = mfma_bf16(a, b[qt][h], acc[dt]);
        },
        work);
  };

  // the two roles run separate copies of the loop (the same barriers in the
  // same order), so that each copy's registers are allocated on their own
  auto walk = [&](auto role) {
    constexpr bool kDK = decltype(role)::value;
    int cur = lq.head;
    if (cur != INT_MAX) {
      load(cur, 0);
      if (wave == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70 | kTileOps);   // vmcnt(kTileOps): lse, D landed
        lse_to_exp2(0);
      }
    }
    for (int s = 0; cur != INT_MAX; ++s) {
      ++lq.i;
      lq.settle();
      const int next = lq.head;
      wait_vmcnt0();                 // this wavefront's loads of cur have landed
      __syncthreads();               // ... everyone's, and the other buffers are free
      if (next != INT_MAX) load(next, (s + 1) & 1);
      const int qb = lds0 + (s & 1) * T::kBytes;
      const int gb = lds0 + (2 + (s & 1)) * T::kBytes;
      const float* Ls = (const float*)(vec + (s & 1) * 256);
      const float* Ds = (const float*)(vec + 512 + (s & 1) * 256);
      bf16x8 b[2][2];                // dV side: P; dK side: dS
      if constexpr (!kDK) {
        // phase 1: S, then p = exp2(S scale log2(e) - lse log2(e)); the
        // weights of queries 0-31 are computed in the slots of queries 32-63.
        // Pad keys need no mask: a key's weights only reach its own column
        // of the results, which is not stored (natural layout) or stored as
        // zeros (blocked layout).
        f32x16 sacc[2];
        f32x4 l4[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i) l4[qt][i] = *(const f32x4*)(Ls + 32 * qt + 8 * i + 4 * hl);
        auto weights = [&](int qt, int e) {   // elements e, e + 1 of S(qt)
          const float x0 = __builtin_amdgcn_exp2f(
              fmaf(sacc[qt][e], scale_log2, -l4[qt][e >> 2][e & 3]));
          const float x1 = __builtin_amdgcn_exp2f(
              fmaf(sacc[qt][e + 1], scale_log2, -l4[qt][e >> 2][(e & 3) + 1]));
          b[qt][e >> 3][e & 7] = (__bf16)x0;
          b[qt][e >> 3][(e & 7) + 1] = (__bf16)x1;
        };
        rows_slots(qb, sacc, [&](int i) {
          if (i >= A::kSteps) {
            constexpr int kPer = 16 / A::kSteps;   // elements per slot
#pragma unroll
            for (int e = 0; e < kPer; e += 2) weights(0, (i - A::kSteps) * kPer + e);
          }
        });
#pragma unroll
        for (int e = 0; e < 16; e += 2) weights(1, e);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int h = 0; h < 2; ++h) *(bf16x8*)(pbuf + pslot + (2 * qt + h) * 1024) = b[qt][h];
        lds_barrier();               // P of this step is in LDS
        // phase 2: dV^T += dO^T P
        cols_slots(gb, b, [&](int) {});
        if (wave == 0 && next != INT_MAX) {
          __builtin_amdgcn_s_waitcnt(0x0F70 | kTileOps);
          lse_to_exp2((s + 1) & 1);
        }
      } else {
        // phase 1: dP - D, the rows of queries 0-31 in the slots of 32-63
        f32x16 dpacc[2];
        f32x4 d4[2][4];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int i = 0; i < 4; ++i) d4[qt][i] = *(const f32x4*)(Ds + 32 * qt + 8 * i + 4 * hl);
        float dpm[2][16];
        rows_slots(gb, dpacc, [&](int i) {
          if (i >= A::kSteps) {
            constexpr int kPer = 16 / A::kSteps;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
              const int el = (i - A::kSteps) * kPer + e;
              dpm[0][el] = dpacc[0][el] - d4[0][el >> 2][el & 3];
            }
          }
        });
#pragma unroll
        for (int el = 0; el < 16; ++el) dpm[1][el] = dpacc[1][el] - d4[1][el >> 2][el & 3];
        lds_barrier();               // P of this step is in LDS
        // phase 2: dS = P (dP - D); dK^T += Q^T dS.  dS of queries 32-63 is
        // formed in the slots of 0-31.
        bf16x8 p8[2][2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int h = 0; h < 2; ++h) p8[qt][h] = *(const bf16x8*)(pbuf + pslot + (2 * qt + h) * 1024);
        auto ds = [&](int qt, int e) {
          b[qt][e >> 3][e & 7] = (__bf16)((float)p8[qt][e >> 3][e & 7] * dpm[qt][e]);
        };
#pragma unroll
        for (int e = 0; e < 16; ++e) ds(0, e);
        cols_slots(qb, b, [&](int i) {
          constexpr int kHalf = 2 * A::kDTiles;      // slots of queries 0-31
          if (i < kHalf) {
            constexpr int kPer = 16 / kHalf;
#pragma unroll
            for (int e = 0; e < kPer; ++e) ds(1, i * kPer + e);
          }
        });
      }
      cur = next;
    }
  };
  if (dk_side) walk(std::true_type{});
  else walk(std::false_type{});

  if (kvalid || g.layout == 1) {
    __bf16* dst = (dk_side ? dK : dV) + koff;
    if (!kvalid) {                   // pad key of the blocked layout: zeros
#pragma unroll
      for (int t = 0; t < A::kDTiles; ++t) acc[t] = f32x16{};
    }
    store_row<D>(dst, acc, dk_side ? scale : 1.0f, hl);
  }
}

// ---------------------------------------------------------------------------
// float32 kernels: two threads per token (lanes 2t, 2t + 1 hold the two
// channel halves, dot products are completed with one lane exchange), fp32
// FMA, tiles in LDS
// ---------------------------------------------------------------------------
// dQ and D: one workgroup (128 threads) per query block, K and V tiles in LDS.
template <int D>
__global__ void __launch_bounds__(128)
attn_bwd_dq_f32_kernel(const Geo g, const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const float* __restrict__ O,
                       const float* __restrict__ dO, const float* __restrict__ lse,
                       const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
                       float scale, float* __restrict__ dQ, float* __restrict__ delta) {
  constexpr int H = D / 2;                 // channels per thread
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Kt = smem_f;
  float* Vt = smem_f + kN * D;
  const int nb = g.nb;
  const int64_t head = blockIdx.x / nb;
  const int qb = (int)(blockIdx.x - head * nb);
  const int s = threadIdx.x >> 1, c0 = (threadIdx.x & 1) * H;
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);
  const BlockCoord qc = block_coord(g, qb);
  const bool qvalid = (s >> 3) < block_rows_valid(g, qc) && (s & 7) < block_cols_valid(g, qc);
  const int64_t qoff = hoff + block_base(g, qb, qc) + (s >> 3) * row_step + (s & 7) * D + c0;

  float qv[H], dov[H], acc[H];
  float Dq = 0.f;
#pragma unroll
  for (int c = 0; c < H; ++c) {
    qv[c] = qvalid ? Q[qoff + c] : 0.f;
    dov[c] = qvalid ? dO[qoff + c] : 0.f;
    Dq = fmaf(dov[c], qvalid ? O[qoff + c] : 0.f, Dq);
    acc[c] = 0.f;
  }
  Dq += __shfl_xor(Dq, 1);
  const int64_t slot = (head * nb + qb) * kN + s;
  if ((threadIdx.x & 1) == 0) delta[slot] = Dq;
  const float l = lse[slot];
  const bool live = qvalid && l > -INFINITY;
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
    for (int i = threadIdx.x; i < kN * D / 4; i += 128) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if ((r >> 3) < rv && (r & 7) < cv) {
        const int64_t off = base + (r >> 3) * row_step + (r & 7) * D + 4 * c4;
        kv = *(const f32x4*)(K + off);
        vv = *(const f32x4*)(V + off);
      }
      *(f32x4*)(Kt + r * D + 4 * c4) = kv;
      *(f32x4*)(Vt + r * D + 4 * c4) = vv;
    }
    __syncthreads();
    for (int r = 0; r < kN; ++r) {     // both lanes of a pair take the same branches
      if (!((r >> 3) < rv && (r & 7) < cv)) continue;
      float dot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < H; ++c) {
        dot = fmaf(qv[c], Kt[r * D + c0 + c], dot);
        dp = fmaf(dov[c], Vt[r * D + c0 + c], dp);
      }
      dot += __shfl_xor(dot, 1);
      dp += __shfl_xor(dp, 1);
      const float ds = live ? expf(dot * scale - l) * (dp - Dq) : 0.f;
#pragma unroll
      for (int c = 0; c < H; ++c) acc[c] = fmaf(ds, Kt[r * D + c0 + c], acc[c]);
    }
  }
  if (qvalid || g.layout == 1) {
#pragma unroll
    for (int c = 0; c < H; ++c) dQ[qoff + c] = qvalid ? acc[c] * scale : 0.f;
  }
}

// dK (threads 128-255) and dV (threads 0-127), two threads per key: one
// workgroup per key block, the Q and dO tiles of each listed query block in
// LDS.
template <int D>
__global__ void __launch_bounds__(256)
attn_bwd_dkdv_f32_kernel(const Geo g, const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, const float* __restrict__ dO,
                         const float* __restrict__ lse, const float* __restrict__ delta,
                         const int32_t* __restrict__ col_ptr, const int32_t* __restrict__ row_idx,
                         float scale, float* __restrict__ dK, float* __restrict__ dV) {
  constexpr int H = D / 2;
  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Qt = smem_f;
  float* Gt = smem_f + kN * D;        // dO tile
  float* Lt = smem_f + 2 * kN * D;    // lse of the tile's queries (-inf: pad)
  float* Dt = Lt + kN;
  const int nb = g.nb;
  const int64_t head = blockIdx.x / nb;
  const int kb = (int)(blockIdx.x - head * nb);
  const int s = (threadIdx.x & 127) >> 1, c0 = (threadIdx.x & 1) * H;
  const bool dk_side = threadIdx.x >= 128;   // wavefront-uniform
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);
  const BlockCoord kc = block_coord(g, kb);
  const bool kvalid = (s >> 3) < block_rows_valid(g, kc) && (s & 7) < block_cols_valid(g, kc);
  const int64_t koff = hoff + block_base(g, kb, kc) + (s >> 3) * row_step + (s & 7) * D + c0;

  float kv[H], vv[H], acc[H];
#pragma unroll
  for (int c = 0; c < H; ++c) {
    kv[c] = kvalid ? K[koff + c] : 0.f;
    vv[c] = kvalid && dk_side ? V[koff + c] : 0.f;
    acc[c] = 0.f;
  }
  const int32_t* cp = col_ptr + head * (nb + 1);
  const int32_t* rows = row_idx + head * (int64_t)nb * nb;
  const int begin = cp[kb];
  int end = cp[kb + 1];
  if (begin < 0 || end < begin || end > nb * nb) end = begin;
  for (int idx = begin; idx < end; ++idx) {
    const int alpha = rows[idx];
    if ((unsigned)alpha >= (unsigned)nb) continue;
    const BlockCoord ac = block_coord(g, alpha);
    const int rv = block_rows_valid(g, ac), cv = block_cols_valid(g, ac);
    const int64_t base = hoff + block_base(g, alpha, ac);
    __syncthreads();
    for (int i = threadIdx.x; i < kN * D / 4; i += 256) {
      const int r = i / (D / 4), c4 = i % (D / 4);
      f32x4 qq = {0.f, 0.f, 0.f, 0.f}, gg = {0.f, 0.f, 0.f, 0.f};
      if ((r >> 3) < rv && (r & 7) < cv) {
        const int64_t off = base + (r >> 3) * row_step + (r & 7) * D + 4 * c4;
        qq = *(const f32x4*)(Q + off);
        gg = *(const f32x4*)(dO + off);
      }
      *(f32x4*)(Qt + r * D + 4 * c4) = qq;
      *(f32x4*)(Gt + r * D + 4 * c4) = gg;
    }
    if (threadIdx.x < kN) {
      Lt[threadIdx.x] = lse[(head * nb + alpha) * kN + threadIdx.x];
      Dt[threadIdx.x] = delta[(head * nb + alpha) * kN + threadIdx.x];
    }
    __syncthreads();
    for (int r = 0; r < kN; ++r) {     // both lanes of a pair take the same branches
      if (!((r >> 3) < rv && (r & 7) < cv) || !(Lt[r] > -INFINITY)) continue;
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < H; ++c) dot = fmaf(Qt[r * D + c0 + c], kv[c], dot);
      dot += __shfl_xor(dot, 1);
      const float p = kvalid ? expf(dot * scale - Lt[r]) : 0.f;
      if (dk_side) {
        float dp = 0.f;
#pragma unroll
        for (int c = 0; c < H; ++c) dp = fmaf(Gt[r * D + c0 + c], vv[c], dp);
        dp += __shfl_xor(dp, 1);
        const float ds = p * (dp - Dt[r]);
#pragma unroll
        for (int c = 0; c < H; ++c) acc[c] = fmaf(ds, Qt[r * D + c0 + c], acc[c]);
      } else {
#pragma unroll
        for (int c = 0; c < H; ++c) acc[c] = fmaf(p, Gt[r * D + c0 + c], acc[c]);
      }
    }
  }
  if (kvalid || g.layout == 1) {
    float* dst = (dk_side ? dK : dV) + koff;
    const float mul = kvalid ? (dk_side ? scale : 1.0f) : 0.f;
#pragma unroll
    for (int c = 0; c < H; ++c) dst[c] = acc[c] * mul;
  }
}

template <int D>
hipError_t launch_dq_t(const Geo& g, bool bf16, const void* q, const void* k, const void* v,
                       const void* o, const void* dout, const float* lse, const int32_t* row_ptr,
                       const int32_t* col_idx, float scale, void* dq, float* delta,
                       hipStream_t s) {
  if (bf16) {
    const int64_t chunk = (pair_items(g) + 7) / 8;
    const size_t lds = 4 * SwTile<D>::kBytes;
    auto kern = attn_bwd_dq_kernel<D>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * chunk * g.bh)), dim3(256), lds, s,
                       g, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)o,
                       (const __bf16*)dout, lse, row_ptr, col_idx, scale * kLog2e, scale,
                       (__bf16*)dq, delta);
    return hipGetLastError();
  }
  const size_t lds = 2 * kN * D * sizeof(float);
  auto kern = attn_bwd_dq_f32_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(g.bh * g.nb)), dim3(128), lds, s, g, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)o, (const float*)dout, lse,
                     row_ptr, col_idx, scale, (float*)dq, delta);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_t(const Geo& g, bool bf16, const void* q, const void* k, const void* v,
                         const void* dout, const float* lse, const float* delta,
                         const int32_t* col_ptr, const int32_t* row_idx, float scale, void* dk,
                         void* dv, hipStream_t s) {
  if (bf16) {
    const int64_t chunk = (g.nb + 7) / 8;
    const size_t lds = 4 * SwTile<D>::kBytes + 4 * 256 + 8192;
    auto kern = attn_bwd_dkdv_kernel<D>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(8 * chunk * g.bh)), dim3(256), lds, s, g,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout,
                       lse, delta, col_ptr, row_idx, scale * kLog2e, scale, (__bf16*)dk,
                       (__bf16*)dv);
    return hipGetLastError();
  }
  const size_t lds = (2 * kN * D + 2 * kN) * sizeof(float);
  auto kern = attn_bwd_dkdv_f32_kernel<D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(g.bh * g.nb)), dim3(256), lds, s, g, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)dout, lse, delta, col_ptr,
                     row_idx, scale, (float*)dk, (float*)dv);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask_transpose(const Geo& g, const uint32_t* bits, uint32_t* bits_t,
                                 int32_t* count_t, hipStream_t s) {
  hipLaunchKernelGGL(mask_transpose_kernel, dim3((unsigned)g.nb, (unsigned)g.bh), dim3(64), 0, s,
                     g, bits, bits_t, count_t);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_dq(const Geo& g, bool bf16, const void* q, const void* k,
                              const void* v, const void* o, const void* dout, const float* lse,
                              const int32_t* row_ptr, const int32_t* col_idx, float scale,
                              void* dq, float* delta, hipStream_t s) {
  return g.d == 64 ? launch_dq_t<64>(g, bf16, q, k, v, o, dout, lse, row_ptr, col_idx, scale, dq,
                                     delta, s)
                   : launch_dq_t<128>(g, bf16, q, k, v, o, dout, lse, row_ptr, col_idx, scale, dq,
                                      delta, s);
}

hipError_t launch_attn_bwd_dkdv(const Geo& g, bool bf16, const void* q, const void* k,
                                const void* v, const void* dout, const float* lse,
                                const float* delta, const int32_t* col_ptr,
                                const int32_t* row_idx, float scale, void* dk, void* dv,
                                hipStream_t s) {
  return g.d == 64 ? launch_dkdv_t<64>(g, bf16, q, k, v, dout, lse, delta, col_ptr, row_idx, scale,
                                       dk, dv, s)
                   : launch_dkdv_t<128>(g, bf16, q, k, v, dout, lse, delta, col_ptr, row_idx,
                                        scale, dk, dv, s);
}

}  // namespace nabla
