// Block-sparse attention forward, bf16, V given as V^T tiles
// ("NABLA: Neighborhood Adaptive Block-Level Attention", gist.science,
// Methodology: expansion of the block mask back to token resolution;
// lsdiaocha.cn article, sec. 2 step 3: each kept reduced entry stands for a
// whole N x N block computed exactly).
//
// One workgroup (4 wavefronts) serves a PAIR of query blocks that see similar
// keys (the same 8x8 patch in two consecutive frames; an odd last frame pairs
// horizontal neighbours) and walks the ascending union of their kept lists,
// so every K / V^T tile of the union is brought on chip once for both.
// Wavefronts 0-1 own the first query block, 2-3 the second, 32 queries each.
//
// Dense mode (nabla_dense_attn_fwd; full attention, the baseline the method's
// speed-ups are quoted against -- gist.science page, experimental results 1):
// the same loop with eight wavefronts serving four consecutive query blocks,
// the schedule being every key block in order (no lists, no merge, no
// skipped stage).
//
// Prologue: the two kept lists are merged into an LDS list of 16-bit
// entries (block index | latent-edge block << 12 | in-first-list << 14 |
// in-second-list << 15) via LDS bitmaps, so the main loop reads its schedule
// from LDS instead of chasing list pointers, and full blocks skip the edge
// logic.
//
// Main loop, software-pipelined per wavefront.  Stage A(j) = S^T(j) = K(j) Q^T
// on the matrix cores plus the row max of S(j); stage B(j) = online-softmax
// exponentials of S(j) and O^T += V^T(j) P^T(j).  Iteration s runs A(s+1) and
// B(s) interleaved -- the QK matrix instructions of block s+1 execute while
// the exponentials of block s are computed, the PV instructions of block s
// while the max of block s+1 is taken -- so the matrix cores and the vector
// ALU work side by side inside one wavefront.  A wavefront whose query block
// does not keep a block skips that stage's matrix instructions.
//
// Tiles move global -> LDS by direct-to-LDS buffer loads (no register
// staging) into two K and two V^T buffers.  Iteration s loads K(s+2) and
// V^T(s+1) into the buffers that iteration s-1 finished with; one barrier per
// iteration separates consumers and producers.  Tile rows are stored with
// their 16-byte chunks permuted (layouts below) so that each LDS read cycle
// hits distinct banks.
//
// Softmax: S^T orientation, so a lane owns one query and 32 of its 64 keys;
// the row max needs one lane <-> lane^32 exchange (v_permlane32_swap), the
// row sum none until the end.  The running max moves only when a block's max
// exceeds it by more than 8 in the exp2 domain, a factor of 2^8 (exact: O
// and the row sum share the reference).  The row sum adds the bf16-ROUNDED
// weights, so O / l is an exact convex combination of the V rows the matrix
// cores saw.  Pad key rows of latent-edge blocks load row 0 of the block (a
// real key, so the block max is unchanged) and get weight 0; pad queries are
// not written in the natural layout and are written as zeros in the blocked
// layout.
#include <type_traits>

#include "attn_common.hpp"

namespace nabla {

namespace {

// LDS tile layouts.  Reads of 16-byte operand chunks are served 16 lanes
// (16 consecutive tile rows, one logical chunk) per cycle, so a layout must
// put those 16 rows in 16 distinct 4-bank groups:
//  * 128-byte rows (V^T tiles; K tiles at d = 64): physical chunk = logical
//    chunk ^ g(r), g(r) = (r & 7) ^ ((r >> 3) & 1); two rows share a 256-byte
//    bank line, and g differs across each 8-row half.
//  * 256-byte rows (K tiles at d = 128): physical chunk = logical ^ (r & 7),
//    and 128 bytes of padding after every 8 rows move rows 8-15 into the other
//    half of the banks.  Each 8-row group is 2 KB contiguous, so tiles still
//    fill in whole 1-KB direct loads.
template <int D, int NW>
struct VtShape {
  static constexpr bool kWideK = D == 128;             // 256-byte K rows
  static constexpr int kKGroupBytes = kWideK ? 8 * 256 + 128 : 8 * 128;
  static constexpr int kKBytes = 8 * kKGroupBytes;     // K tile in LDS
  static constexpr int kVBytes = D * kN * 2;           // V^T tile: d rows x 128 bytes
  static constexpr int kKChunks = D / 8;               // 16-byte chunks per K row
  static constexpr int kKOps = kN * D * 2 / 1024 / NW;  // 1-KB direct loads per wavefront
  static constexpr int kVOps = kVBytes / 1024 / NW;
  static constexpr int kSteps = D / 16;                // k-steps of S^T = K Q^T
  static constexpr int kDTiles = D / 32;               // 32-row tiles of O^T
  static constexpr int kBufBytes = 2 * kKBytes + 2 * kVBytes;
  // LDS byte offset of direct load op o within a K tile
  __device__ static int k_op_offset(int o) {
    return kWideK ? (o >> 1) * kKGroupBytes + (o & 1) * 1024 : o * 1024;
  }
};

__device__ inline int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// schedule entry flag: the block overhangs the latent edge (pad rows or columns)
constexpr int kEdgeBit = 1 << 12;

__device__ inline float swap_max(float x) {   // max over lanes l and l ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, typename OutT, int NW, bool kDense>
__global__ void __launch_bounds__(NW * 64, 8 / NW)
attn_fwd_vt_kernel(const Geo g, const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ VT, const int32_t* __restrict__ row_ptr,
                   const int32_t* __restrict__ col_idx, float scale_log2,
                   OutT* __restrict__ O, float* __restrict__ lse) {
  static_assert(kDense || NW == 4, "the sparse walk serves pairs of query blocks");
  constexpr int QB = NW / 2;         // query blocks per workgroup
  using S = VtShape<D, NW>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  char* const kbuf = smem;                          // [2][kKBytes]
  char* const vbuf = smem + 2 * S::kKBytes;         // [2][kVBytes]
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  uint32_t* const bm = (uint32_t*)(smem + S::kBufBytes);   // [2][nw] bitmaps, then the count
  uint16_t* const ul = (uint16_t*)(bm + 2 * nw + 1);       // union list [nb]

  const int items = kDense ? (nb + QB - 1) / QB : pair_items(g);
  int64_t head;
  int item;
  if (!xcd_item(blockIdx.x, items, (items + 7) >> 3, &head, &item)) return;
  int qa = -1, qpair = -1;
  if constexpr (!kDense) pair_of(g, item, &qa, &qpair);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 1;         // query block of the workgroup (sparse: of the pair)
  const int hl = lane >> 5;          // lane half
  const int jl = lane & 31;          // query column / operand row of this lane
  // -1: this wavefront only helps load
  const int myq = kDense ? (QB * item + grp < nb ? QB * item + grp : -1)
                         : (grp == 0 ? qa : qpair);
  const int64_t hoff = head * (int64_t)g.head_elems;
  const int row_step = block_row_step(g);

  if constexpr (kDense) {
    // ---- every key block, in order ----
    for (int j = tid; j < nb; j += NW * 64) {
      const BlockCoord c = block_coord(g, j);
      const bool edge = block_rows_valid(g, c) < kP || block_cols_valid(g, c) < kP;
      ul[j] = (uint16_t)(j | ((int)edge << 12) | (3 << 14));
    }
    if (tid == 0) bm[2 * nw] = (uint32_t)nb;
    __syncthreads();
  } else {
    // ---- merged schedule: LDS bitmaps of both lists -> ascending union ----
    for (int w = tid; w < 2 * nw; w += NW * 64) bm[w] = 0u;
    __syncthreads();
    {
      const int32_t* rp = row_ptr + head * (nb + 1);
      const int32_t* cols = col_idx + head * (int64_t)nb * nb;
  #pragma unroll
      for (int l = 0; l < 2; ++l) {
        const int q = l == 0 ? qa : qpair;
        if (q < 0) continue;
        const int begin = rp[q], end = rp[q + 1];
        if (begin < 0 || end < begin || end > nb * nb) continue;   // malformed row: no keys
        for (int i = begin + tid; i < end; i += NW * 64) {
          const int c = cols[i];
          if ((unsigned)c < (unsigned)nb) atomicOr(&bm[l * nw + (c >> 5)], 1u << (c & 31));
        }
      }
    }
    __syncthreads();
    if (wave == 0) {                   // nw <= 128: two words per lane
      const int w0 = 2 * lane, w1 = w0 + 1;
      const uint32_t a0 = w0 < nw ? bm[w0] : 0u, b0 = w0 < nw ? bm[nw + w0] : 0u;
      const uint32_t a1 = w1 < nw ? bm[w1] : 0u, b1 = w1 < nw ? bm[nw + w1] : 0u;
      const int cnt = __popc(a0 | b0) + __popc(a1 | b1);
      int incl = cnt;
  #pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      int pos = incl - cnt;
      auto expand = [&](uint32_t a, uint32_t b, int w) {
        uint32_t u = a | b;
        while (u) {
          const int bit = __builtin_ctz(u);
          u &= u - 1;
          const int blk = (w << 5) | bit;
          const BlockCoord c = block_coord(g, blk);
          const bool edge = block_rows_valid(g, c) < kP || block_cols_valid(g, c) < kP;
          ul[pos++] = (uint16_t)(blk | ((int)edge << 12) | (((a >> bit) & 1u) << 14) |
                                 (((b >> bit) & 1u) << 15));
        }
      };
      expand(a0, b0, w0);
      expand(a1, b1, w1);
      if (lane == 63) bm[2 * nw] = (uint32_t)incl;
    }
    __syncthreads();
  }
  const int U = __builtin_amdgcn_readfirstlane((int)bm[2 * nw]);
  const int mine_bit = 14 + grp;     // flag of this wavefront's query block in an entry
  // does this wavefront's query block keep the entry's key block
  auto mine = [&](int e) { return kDense ? e >= 0 : e >= 0 && ((e >> mine_bit) & 1); };
  auto entry = [&](int j) -> int {   // wave-uniform schedule entry, -1 past the end
    return j < U ? __builtin_amdgcn_readfirstlane((int)ul[j]) : -1;
  };

  // ---- this lane's query row as the B operand of S^T = K Q^T ----
  const int qs = 32 * (wave & 1) + jl;   // slot in the query block
  // offset of this lane's query row in Q and O (recomputed for the epilogue
  // rather than kept live through the loop)
  auto query_row = [&](bool* valid) -> int64_t {
    *valid = false;
    if (myq < 0) return 0;
    const BlockCoord qc = block_coord(g, myq);
    *valid = (qs >> 3) < block_rows_valid(g, qc) && (qs & 7) < block_cols_valid(g, qc);
    return hoff + block_base(g, myq, qc) + (qs >> 3) * row_step + (qs & 7) * D;
  };
  bool qvalid;
  const int64_t qoff = query_row(&qvalid);
  bf16x8 qop[S::kSteps];
#pragma unroll
  for (int s = 0; s < S::kSteps; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qvalid) raw = *(const u32x4*)(Q + qoff + 16 * s + 8 * hl);
    qop[s] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- loop-invariant addressing ----
  // direct loads: K op i of this lane moves tile row r, logical chunk c
  auto kdma_rc = [&](int i, int* r, int* c) {
    const int o = wave * S::kKOps + i;
    if constexpr (S::kWideK) {       // 4 rows of 16 chunks per op
      *r = 4 * o + (lane >> 4);
      *c = (lane & 15) ^ (*r & 7);
    } else {                         // 8 rows of 8 chunks per op
      *r = 8 * o + (lane >> 3);
      *c = (lane & 7) ^ swz128(*r);
    }
  };
  // full-block offset of op i = kdma_lane[i & 1] + kdma_rows(i) * row_step:
  // the op's 8-row group is uniform, its row-in-group and chunk depend on
  // the lane and the op's parity only
  int kdma_lane[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    int r, c;
    kdma_rc(par, &r, &c);
    kdma_lane[par] = (r & 7) * D + c * 8;
  }
  auto kdma_rows = [&](int i) {     // 8-row group of op i (wavefront-uniform)
    return S::kWideK ? (S::kKOps / 2) * wave + (i >> 1) : S::kKOps * wave + i;
  };
  auto kdma_full = [&](int i) { return kdma_rows(i) * row_step + kdma_lane[i & 1]; };
  // V^T op o: rows 8o + lane / 8, logical chunk (lane % 8) ^ g(row); g's
  // bit from row bit 3 equals o & 1, so even and odd ops differ
  int vdma[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int r = 8 * (wave * S::kVOps + par) + (lane >> 3);
    vdma[par] = r * kN + (((lane & 7) ^ swz128(r)) << 3) - par * 512;
  }
  // LDS operand reads (bytes within a tile).  Rows 32t + jl share their low
  // 4 bits with jl, so the tile index t only adds a constant; logical chunk
  // 2s + hl lands at physical 2(s ^ y) + z, so four lane addresses plus
  // immediate offsets cover every read.
  // absolute LDS addresses (K buffer 0 / V^T buffer 0), so that each read
  // is a register plus an immediate offset
  const int lds0 = (int)(uintptr_t)(lds_char*)smem;
  int kaddr[4], vaddr[4];
  {
    const int gk = S::kWideK ? (jl & 7) : swz128(jl);
    const int gv = swz128(jl);
    const int kbase = S::kWideK ? (jl >> 3) * S::kKGroupBytes + (jl & 7) * 256 : jl * 128;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      kaddr[q] = lds0 + kbase + (((2 * q + hl) ^ gk) << 4);
      vaddr[q] = lds0 + 2 * S::kKBytes + jl * 128 + (((2 * q + hl) ^ gv) << 4);
    }
  }
  auto kread = [&](int kt, int s) {  // K row 32kt + jl, logical chunk 2s + hl
    if constexpr (S::kWideK)          // chunk bit 3 (s >= 4) is never swizzled: +128 bytes
      return kaddr[s & 3] + (s >> 2) * 128 + kt * 4 * S::kKGroupBytes;
    else
      return kaddr[s] + kt * 32 * 128;
  };
  auto vread = [&](int dt, int i) { return vaddr[i] + dt * 32 * 128; };

  // one descriptor per head and tensor: byte offsets within a head fit in 32
  // bits (a head holds fewer than 2^31 elements)
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(K + hoff, 2u * (uint32_t)g.head_elems);
  const __amdgpu_buffer_rsrc_t vrs =
      buffer_rsrc(VT + head * nb * (int64_t)(kN * D), 2u * (uint32_t)(nb * kN * D));
  uint32_t kdma_voff[2], vdma_voff[2];   // per-lane byte offsets
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    kdma_voff[par] = 2u * (uint32_t)kdma_lane[par];
    vdma_voff[par] = 2u * (uint32_t)vdma[par];
  }
  auto load_k = [&](int e, char* dst) {
    const int beta = e & 0xFFF;
    const BlockCoord bc = block_coord(g, beta);
    const uint32_t sb = 2u * (uint32_t)block_base(g, beta, bc);
    if (!(e & kEdgeBit)) {           // lane part in the vector offset, the rest scalar
#pragma unroll
      for (int i = 0; i < S::kKOps; ++i)
        dma16(krs, kdma_voff[i & 1], sb + 2u * (uint32_t)(kdma_rows(i) * row_step),
              dst + S::k_op_offset(wave * S::kKOps + i));
    } else {                         // pad rows re-read row 0 of the block
      const int rv = block_rows_valid(g, bc);
      const int cv = block_cols_valid(g, bc);
#pragma unroll
      for (int i = 0; i < S::kKOps; ++i) {
        int r, c;
        kdma_rc(i, &r, &c);
        const bool ok = (r >> 3) < rv && (r & 7) < cv;
        dma16(krs, 2u * (uint32_t)(ok ? kdma_full(i) : c * 8), sb,
              dst + S::k_op_offset(wave * S::kKOps + i));
      }
    }
  };
  auto load_v = [&](int e, char* dst) {
    const uint32_t sb = 2u * (uint32_t)((e & 0xFFF) * (kN * D));
#pragma unroll
    for (int i = 0; i < S::kVOps; ++i)
      dma16(vrs, vdma_voff[i & 1], sb + 1024u * i, dst + (wave * S::kVOps + i) * 1024);
  };

  f32x16 oacc[S::kDTiles];
#pragma unroll
  for (int t = 0; t < S::kDTiles; ++t) oacc[t] = f32x16{};
  // running max (exp2 domain) of this lane's query; a finite start keeps a
  // block whose keys are all masked at p = exp2(-inf) = 0
  float m_run = -1e30f;
  float l_run = 0.f;                 // partial row sum over the keys this lane holds
  float mx_cur = -INFINITY;          // max (exp2 domain) of the block B works on next
  float mx_next = -INFINITY;

  // B(j) preparation on entry: lazy rescale, pad-key masking
  auto stage_b_pre = [&](f32x16 (&sc)[2], int e) {
    if (__builtin_amdgcn_ballot_w64(mx_cur > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx_cur);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first block
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < S::kDTiles; ++t) oacc[t] *= alpha;
      m_run = m_new;
    }
    if (e & kEdgeBit) {              // element r of sc[kt]: key row 4kt + r/4, column 4hl + r%4
      const BlockCoord bc = block_coord(g, e & 0xFFF);
      const int rv = block_rows_valid(g, bc);
      const int cv = block_cols_valid(g, bc);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (!((4 * kt + (r >> 2)) < rv && (4 * hl + (r & 3)) < cv)) sc[kt][r] = -INFINITY;
    }
  };

  // exponentials of elements r, r + 1 of sc[kt] into the bf16 operand P^T;
  // the row sum adds the rounded values (bf16 pairs summed by v_dot2_f32_bf16)
  // (m_ref = +inf gives exact zeros: scores are always finite here).  The
  // slot's scheduling barrier keeps this work in its slot; inside the slot
  // the compiler puts the operand read between the exponentials and their
  // first use, which the transcendental-result hazard would otherwise fill
  // with a wait state.
  auto exp_pair = [&](const f32x16 (&sc)[2], bf16x8 (&pop)[2][2], int kt, int r, float m_ref) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    const float x0 = __builtin_fmaf(sc[kt][r], scale_log2, -m_ref);
    const float x1 = __builtin_fmaf(sc[kt][r + 1], scale_log2, -m_ref);
    const bf16x2 pr = {(__bf16)__builtin_amdgcn_exp2f(x0), (__bf16)__builtin_amdgcn_exp2f(x1)};
    l_run = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run, false);
    pop[kt][r >> 3][r & 7] = pr[0];
    pop[kt][r >> 3][(r & 7) + 1] = pr[1];
  };

  // One iteration's work: A(s+1) on K buffer kb (if DoA), B(s) on V^T buffer
  // vb (if DoB); sc holds S(s) (consumed), sn receives S(s+1).  Written as
  // slots -- one matrix instruction, its share of vector work, one operand
  // read 3 slots ahead -- fenced so the compiler keeps that order: QK slots
  // carry the exponentials of B(s), PV slots the row max of A(s+1).
  auto body = [&](auto do_a, auto do_b, bool run_a, bool live_b, f32x16 (&sc)[2],
                  f32x16 (&sn)[2], int kb, int vb) {
    constexpr bool DoA = decltype(do_a)::value;
    constexpr bool DoB = decltype(do_b)::value;
    constexpr int NQ = DoA ? 2 * S::kSteps : 0;      // QK matrix instructions
    constexpr int NP = DoB ? 4 * S::kDTiles : 0;     // PV matrix instructions
    constexpr int NR = NQ + NP;                      // operand reads, K then V^T
    constexpr int kAhead = NR < 3 ? NR : 3;
    bf16x8 op[NR > 0 ? NR : 1];
    auto read = [&](int j) {
      if (j < NQ)
        op[j] = lds_read16(kb + kread(j & 1, j >> 1));
      else
        op[j] = lds_read16(vb + vread((j - NQ) % S::kDTiles, (j - NQ) / S::kDTiles));
    };
#pragma unroll
    for (int j = 0; j < kAhead; ++j) read(j);
    bf16x8 pop[2][2];
    // a block this wavefront does not keep enters with weight exactly 0
    const float m_ref = live_b ? m_run : INFINITY;
    if constexpr (DoA) {
      constexpr int kExpPerSlot = 32 / (NQ > 0 ? NQ : 1);   // score elements per QK slot
      // two copies of the QK slots, with and without the matrix instructions
      // (a wavefront that does not keep block s+1 skips them; sn then keeps
      // an older finite score tile, whose max is ignored and whose weights
      // are computed against the reference +inf, i.e. exactly 0)
      auto qk_slots = [&](auto with_mfma) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int kt = i & 1, st = i >> 1;     // the two score tiles alternate
          if constexpr (decltype(with_mfma)::value)
            sn[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op[i], qop[st], st == 0 ? f32x16{} : sn[kt],
                                                             0, 0, 0);
          if constexpr (DoB) {
#pragma unroll
            for (int e = 0; e < kExpPerSlot; e += 2) {
              const int el = i * kExpPerSlot + e;    // element of sc: kt = el / 16, r = el % 16
              exp_pair(sc, pop, el >> 4, el & 15, m_ref);
            }
          }
          if (i + kAhead < NR) read(i + kAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (run_a) qk_slots(std::true_type{});
      else qk_slots(std::false_type{});
    } else if constexpr (DoB) {
#pragma unroll
      for (int el = 0; el < 32; el += 2) exp_pair(sc, pop, el >> 4, el & 15, m_ref);
    }
    float mx = -INFINITY;
    if constexpr (DoB) {
      constexpr int kMaxPerSlot = 32 / NP;           // score elements of sn per PV slot
      // two copies of the PV slots, with and without the matrix instructions
      // (a wavefront that does not keep block s skips them)
      auto pv_slots = [&](auto with_mfma) {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          if constexpr (decltype(with_mfma)::value)
            oacc[i % S::kDTiles] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(   // d tiles rotate
                op[NQ + i], pop[(i / S::kDTiles) >> 1][(i / S::kDTiles) & 1], oacc[i % S::kDTiles], 0, 0, 0);
          if constexpr (DoA) {
#pragma unroll
            for (int e = 0; e < kMaxPerSlot; e += 2) {
              const int el = i * kMaxPerSlot + e;
              mx = fmaxf(mx, fmaxf(sn[el >> 4][el & 15], sn[el >> 4][(el & 15) + 1]));
            }
            asm volatile("" ::"v"(mx));
          }
          if (NQ + i + kAhead < NR) read(NQ + i + kAhead);
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (live_b) pv_slots(std::true_type{});
      else pv_slots(std::false_type{});
    } else if constexpr (DoA) {
#pragma unroll
      for (int el = 0; el < 32; el += 2)
        mx = fmaxf(mx, fmaxf(sn[el >> 4][el & 15], sn[el >> 4][(el & 15) + 1]));
    }
    if constexpr (DoA) mx_next = swap_max(mx) * scale_log2;
  };

  // ---- prologue: K(0), V^T(0), K(1) on chip, A(0) ----
  int e0 = entry(0), e1 = entry(1), e2 = entry(2);
  f32x16 s0[2], s1[2];
  s0[0] = s0[1] = s1[0] = s1[1] = f32x16{};
  if (e0 >= 0) {
    load_k(e0, kbuf);
    load_v(e0, vbuf);
    if (e1 >= 0) load_k(e1, kbuf + S::kKBytes);
  }
  wait_vmcnt0();
  __builtin_amdgcn_s_barrier();
  if (mine(e0)) {
    bf16x8 ka[2][S::kSteps];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < S::kSteps; ++s) ka[kt][s] = lds_read16(kread(kt, s));
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < S::kSteps; ++s)
        s0[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kt][s], qop[s], s0[kt], 0, 0, 0);
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s0[kt][r]);
    mx_cur = swap_max(mx) * scale_log2;
  }

  // ---- iteration s: loads K(s+2), V^T(s+1); runs A(s+1) and B(s) ----
  auto iteration = [&](int s, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    wait_vmcnt0();                   // this wavefront's loads of iteration s-1 have landed
    __builtin_amdgcn_s_barrier();    // ... everyone's, and everyone is done with s-1's buffers
    const int e3v = s + 3 < U ? (int)ul[s + 3] : -1;   // made uniform at the end
    if (e2 >= 0) load_k(e2, kbuf + (s & 1) * S::kKBytes);
    if (e1 >= 0) load_v(e1, vbuf + ((s + 1) & 1) * S::kVBytes);
    const bool do_b = mine(e0);
    const bool do_a = mine(e1);
    if (do_b) stage_b_pre(sc, e0);
    const int kb = ((s + 1) & 1) * S::kKBytes;   // buffer offsets within the K / V^T areas
    const int vb = (s & 1) * S::kVBytes;
    using T = std::true_type;
    // a step with work for either stage runs one body: the matrix
    // instructions of an unneeded stage are skipped, its vector work runs
    // harmlessly (an unneeded max is ignored, unneeded exponentials get the
    // reference +inf and are exactly 0), so all cases share one register
    // layout
    if (do_a || do_b) body(T{}, T{}, do_a, do_b, sc, sn, kb, vb);
    if (do_a) mx_cur = mx_next;
    e0 = e1;
    e1 = e2;
    e2 = __builtin_amdgcn_readfirstlane(e3v);
  };
  for (int s = 0; s < U; s += 2) {
    iteration(s, s0, s1);
    if (s + 1 < U) iteration(s + 1, s1, s0);
  }

  // ---- normalise and write this lane's query row ----
  const float l_tot = swap_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  bool ovalid;
  const int64_t ooff = query_row(&ovalid);
  if (lse != nullptr && myq >= 0 && hl == 0)   // ln sum exp(s * scale) = (m + log2 l) ln 2
    lse[(head * nb + myq) * kN + qs] =
        ovalid && l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
  if (myq >= 0 && (ovalid || g.layout == 1)) {
    OutT* orow = O + ooff;
    const float sc = ovalid ? inv : 0.f;
#pragma unroll
    for (int dt = 0; dt < S::kDTiles; ++dt) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        store4<OutT>(orow + 32 * dt + 8 * gq + 4 * hl, oacc[dt][4 * gq] * sc,
                     oacc[dt][4 * gq + 1] * sc, oacc[dt][4 * gq + 2] * sc,
                     oacc[dt][4 * gq + 3] * sc);
      }
    }
  }
}

template <int D, typename OutT, int NW, bool kDense>
hipError_t launch_vt(const Geo& g, const void* q, const void* k, const void* vt,
                     const int32_t* row_ptr, const int32_t* col_idx, float scale, void* o,
                     float* lse, hipStream_t s) {
  using S = VtShape<D, NW>;
  const int nw = (g.nb + 31) >> 5;
  const size_t lds = S::kBufBytes + (size_t)(2 * nw + 1) * 4 + (size_t)g.nb * 2;
  auto kern = attn_fwd_vt_kernel<D, OutT, NW, kDense>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const float sl2 = scale * 1.4426950408889634f;   // exp(x) = exp2(x log2 e)
  const int64_t items = kDense ? (g.nb + NW / 2 - 1) / (NW / 2) : pair_items(g);
  const int64_t chunk = (items + 7) / 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)(8 * chunk * g.bh)), dim3(NW * 64), lds, s, g,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)vt, row_ptr, col_idx,
                     sl2, (OutT*)o, lse);
  return hipGetLastError();
}

// dense: four query blocks per workgroup (eight wavefronts), every key block
constexpr int kDenseWaves = 8;

}  // namespace

hipError_t launch_attn_fwd_vt(const Geo& g, bool out_bf16, const void* q, const void* k,
                              const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                              float scale, void* o, float* lse, hipStream_t s) {
  if (g.d == 64)
    return out_bf16
               ? launch_vt<64, __bf16, 4, false>(g, q, k, vt, row_ptr, col_idx, scale, o, lse, s)
               : launch_vt<64, float, 4, false>(g, q, k, vt, row_ptr, col_idx, scale, o, lse, s);
  return out_bf16
             ? launch_vt<128, __bf16, 4, false>(g, q, k, vt, row_ptr, col_idx, scale, o, lse, s)
             : launch_vt<128, float, 4, false>(g, q, k, vt, row_ptr, col_idx, scale, o, lse, s);
}

hipError_t launch_attn_dense_vt(const Geo& g, bool out_bf16, const void* q, const void* k,
                                const void* vt, float scale, void* o, float* lse,
                                hipStream_t s) {
  constexpr int NW = kDenseWaves;
  if (g.d == 64)
    return out_bf16
               ? launch_vt<64, __bf16, NW, true>(g, q, k, vt, nullptr, nullptr, scale, o, lse, s)
               : launch_vt<64, float, NW, true>(g, q, k, vt, nullptr, nullptr, scale, o, lse, s);
  return out_bf16
             ? launch_vt<128, __bf16, NW, true>(g, q, k, vt, nullptr, nullptr, scale, o, lse, s)
             : launch_vt<128, float, NW, true>(g, q, k, vt, nullptr, nullptr, scale, o, lse, s);
}

}  // namespace nabla
