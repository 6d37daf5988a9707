// Shared device-side definitions of libnabla (gfx950): geometry of the
// fractal-flattened latent, token addressing in either tensor layout, vector
// types for the matrix cores, and the internal launcher declarations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nabla {

constexpr int kP = 8;          // patch side
constexpr int kN = kP * kP;    // tokens per block

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Geometry of one call.  Blocks are P x P spatial patches of one frame
// ("NABLA: Neighborhood Adaptive Block-Level Attention", gist.science,
// Methodology: token reordering); H and W are padded up to Hp, Wp.
// Division of n < 2^16 by a fixed d <= 2^16 without a divide sequence:
// with m = floor(2^32 / d) + 1 split as (hi, lo) at 2^32,
// n / d == hi * n + ((n * lo) >> 32) exactly (error of n*m/2^32 is < 2^-16 <= 1/d).
struct Recip {
  uint32_t lo;
  uint32_t hi;
};
inline Recip make_recip(uint32_t d) {
  const uint64_t m = (((uint64_t)1) << 32) / d + 1;
  return Recip{(uint32_t)m, (uint32_t)(m >> 32)};
}
__host__ __device__ inline int div16(int n, Recip r) {
  return (int)(r.hi * (uint32_t)n + (uint32_t)(((uint64_t)(uint32_t)n * r.lo) >> 32));
}

struct Geo {
  int64_t bh;        // batch * heads
  int T, H, W;       // valid extents
  int gh, gw;        // block rows / columns per frame (Hp / 8, Wp / 8)
  int nb;            // blocks per head (< 2^16)
  int d;             // head dim
  int layout;        // 0: [.., T, H, W, d]   1: [.., nb, 64, d]
  int head_elems;    // elements per head in the tensor layout (< 2^31)
  Recip per_frame_r; // division by gh * gw
  Recip gw_r;        // division by gw
};

// Pooled keys.  Each float32 mean x is stored exactly as three bf16 parts
// h = bf16(x), m = bf16(x - h), l = x - h - m (x - h and x - h - m are exact
// in float32, and the last one fits in bf16), so h + m + l == x, and the mask
// kernel forms q.k from six bf16 products.  The parts sit in tiles of 16
// blocks in the order of that kernel's matrix-core operand loads: within
// tile j, k-step t (channels 32 t .. 32 t + 31) and part p, lane 16 g + i of a
// wavefront reads the 16 bytes of block 16 j + i, channels 32 t + 8 g .. + 7,
// so each load is one contiguous kilobyte.  Offset in bf16 elements within a
// head, and the padded row count of a head:
__host__ __device__ inline int kbar_rows(int nb) { return (nb + 15) & ~15; }
__host__ __device__ inline int kbar_offset(int row, int c, int p, int d) {
  return ((((row >> 4) * (d >> 5) + (c >> 5)) * 3 + p) * 64 + ((c >> 3) & 3) * 16 + (row & 15)) *
             8 + (c & 7);
}
// bf16 elements of one head's pooled keys
__host__ __device__ inline int64_t kbar_head_elems(int nb, int d) {
  return (int64_t)kbar_rows(nb) * d * 3;
}

struct BlockCoord {
  int t, hb, wb;
};

__host__ __device__ inline BlockCoord block_coord(const Geo& g, int b) {
  BlockCoord c;
  c.t = div16(b, g.per_frame_r);
  const int r = b - c.t * (g.gh * g.gw);
  c.hb = div16(r, g.gw_r);
  c.wb = r - c.hb * g.gw;
  return c;
}

// Raw buffer descriptor over n bytes at p (gfx9 word 3: 32-bit data format).
// Loads at byte offsets >= n return zeros.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

// Valid rows / columns of block b's 8 x 8 patch (8 unless it overhangs the latent edge).
__device__ inline int block_rows_valid(const Geo& g, const BlockCoord& c) {
  const int r = g.H - c.hb * kP;
  return r < kP ? r : kP;
}
__device__ inline int block_cols_valid(const Geo& g, const BlockCoord& c) {
  const int r = g.W - c.wb * kP;
  return r < kP ? r : kP;
}

// Element offset (inside one head) of the first token of block b, and the
// offset step between patch rows; a slot s = i*8 + j of the block sits at
// base + i * row_step + j * d.  In the natural layout the 8 tokens of a patch
// row are contiguous and consecutive patch rows are W tokens apart; in the
// blocked layout the whole block is one contiguous run of 64 tokens.
__device__ inline int block_base(const Geo& g, int b, const BlockCoord& c) {
  if (g.layout == 0) return ((c.t * g.H + c.hb * kP) * g.W + c.wb * kP) * g.d;
  return b * kN * g.d;
}
__device__ inline int block_row_step(const Geo& g) {
  return g.layout == 0 ? g.W * g.d : kP * g.d;
}

// ---------------------------------------------------------------------------
// launchers (each returns the hipError_t of its launch)
// ---------------------------------------------------------------------------
// forward: src natural -> dst blocked; inverse: src blocked -> dst natural
hipError_t launch_flatten(const Geo& g, int elem_bytes, const void* src, void* dst, bool inverse,
                          hipStream_t s);
hipError_t launch_pool(const Geo& g, bool bf16, const void* q, const void* k, float* qbar,
                       __bf16* kbar, hipStream_t s);
hipError_t launch_mask(const Geo& g, const float* qbar, const __bf16* kbar, float thr,
                       const int sta[3], uint32_t* bits, int32_t* cnt, uint32_t* abits,
                       hipStream_t s);
hipError_t launch_compact(const Geo& g, const uint32_t* bits, const int32_t* cnt,
                          int32_t* row_ptr, int32_t* col_idx, hipStream_t s);
// pool, mask and compact in order on one stream (mask.hip)
hipError_t launch_mask_build(const Geo& g, bool bf16, const void* q, const void* k, float* qbar,
                             __bf16* kbar, float thr, const int sta[3], uint32_t* bits,
                             int32_t* cnt, uint32_t* abits, int32_t* row_ptr, int32_t* col_idx,
                             hipStream_t s);
// lse (nullable): float32 [bh, nb, 64] natural-log log-sum-exp of each query's
// scaled scores over its kept valid keys; -inf for pad slots and empty rows
hipError_t launch_attn_fwd(const Geo& g, bool bf16, bool out_bf16, const void* q, const void* k,
                           const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                           float scale, void* o, float* lse, hipStream_t s);
hipError_t launch_transpose_v(const Geo& g, const void* v, void* vt, hipStream_t s);
// gradients (attn_bwd.hip); lse / delta float32 [bh, nb, 64]
hipError_t launch_mask_transpose(const Geo& g, const uint32_t* bits, uint32_t* bits_t,
                                 int32_t* count_t, hipStream_t s);
hipError_t launch_attn_bwd_dq(const Geo& g, bool bf16, const void* q, const void* k,
                              const void* v, const void* o, const void* dout, const float* lse,
                              const int32_t* row_ptr, const int32_t* col_idx, float scale,
                              void* dq, float* delta, hipStream_t s);
hipError_t launch_attn_bwd_dkdv(const Geo& g, bool bf16, const void* q, const void* k,
                                const void* v, const void* dout, const float* lse,
                                const float* delta, const int32_t* col_ptr,
                                const int32_t* row_idx, float scale, void* dk, void* dv,
                                hipStream_t s);
hipError_t launch_attn_fwd_vt(const Geo& g, bool out_bf16, const void* q, const void* k,
                              const void* vt, const int32_t* row_ptr, const int32_t* col_idx,
                              float scale, void* o, float* lse, hipStream_t s);
hipError_t launch_qkv_split(const Geo& g, int batch, int heads, const void* qkv, void* q, void* k,
                            void* vt, float* qbar, __bf16* kbar, hipStream_t s);
hipError_t launch_attn_dense_vt(const Geo& g, bool out_bf16, const void* q, const void* k,
                                const void* vt, float scale, void* o, float* lse,
                                hipStream_t s);

}  // namespace nabla
