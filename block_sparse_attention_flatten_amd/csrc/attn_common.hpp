// Pieces shared by the bf16 attention kernels: the pair work items, the
// workgroup -> (head, item) order, and the output store.
#pragma once

#include <limits.h>

#include "nabla_common.hpp"

namespace nabla {

// Pair work items of one head: item p -> query blocks (a, b), b = -1 when a
// has no partner.  Pairs are (t, hb, wb) and (t + 1, hb, wb) for even t; when
// T is odd the last frame pairs (hb, wb) with (hb, wb + 1) for even wb.
__host__ __device__ inline int pair_items(const Geo& g) {
  const int pf = g.gh * g.gw;
  return (g.T >> 1) * pf + ((g.T & 1) ? g.gh * ((g.gw + 1) >> 1) : 0);
}
__device__ inline void pair_of(const Geo& g, int p, int* a, int* b) {
  const int pf = g.gh * g.gw;
  const int nfull = (g.T >> 1) * pf;
  if (p < nfull) {
    const int t2 = p / pf;
    *a = 2 * t2 * pf + (p - t2 * pf);
    *b = *a + pf;
    return;
  }
  const int q = p - nfull, hw = (g.gw + 1) >> 1;
  const int hb = q / hw, wp = q - hb * hw;
  *a = (g.T - 1) * pf + hb * g.gw + 2 * wp;
  *b = 2 * wp + 1 < g.gw ? *a + 1 : -1;
}

// ---- LDS addressing and direct-to-LDS loads (gfx950) ----
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// 16-byte LDS read at an absolute LDS address
__device__ inline bf16x8 lds_read16(int addr) { return *(lds_bf16x8*)(uintptr_t)addr; }

// s_waitcnt vmcnt(0), leaving the other counters alone.
__device__ inline void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Direct-to-LDS load of 16 bytes per lane through a buffer descriptor: lane
// l reads bytes [soff + voff, +16) of the buffer and writes bytes
// [16 l, 16 l + 16) of the 1-KB LDS block at dst.  The buffer form keeps the
// tile address in scalar registers, and (unlike the global form) does not
// make the compiler drain every outstanding LDS read at each LDS wait.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, char* dst) {
#if defined(__HIP_DEVICE_COMPILE__)   // gfx950-only builtin: the host pass needs no body
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, voff, soff, 0, 0);
#endif
}

// Ascending list of one row of a CSR structure (a query block's kept key
// blocks, or a key block's query blocks in the transposed mask), read through
// the scalar cache (the constant address space makes these uniform reads
// scalar loads); entries outside [0, nb) are skipped so a malformed list
// cannot cause wild reads.
typedef const __attribute__((address_space(4))) int32_t const_i32;
struct KeptList {
  const_i32* p;
  int i, n, nb;
  int head;                          // p[i] (first valid entry from i on), INT_MAX at the end
  __device__ void settle() {
    while (i < n && (unsigned)p[i] >= (unsigned)nb) ++i;
    head = i < n ? p[i] : INT_MAX;
  }
};

__device__ inline KeptList kept_list(const int32_t* row_ptr, const int32_t* cols, int nb, int q) {
  KeptList l = {(const_i32*)cols, 0, 0, nb, INT_MAX};
  if (q < 0) return l;
  const int begin = ((const_i32*)row_ptr)[q];
  const int end = ((const_i32*)row_ptr)[q + 1];
  if (begin < 0 || end < begin || end > nb * nb) return l;   // malformed row: no keys
  l.p = (const_i32*)(cols + begin);
  l.n = end - begin;
  l.settle();
  return l;
}

// Workgroup id -> (head, pair item).  Workgroups are dispatched in id order,
// round-robin over the 8 XCDs (XCD = id % 8).  Each head's items are cut into
// 8 contiguous chunks and XCD x takes chunk (x + h) % 8 of head h: all XCDs
// work on the same head at any time, each XCD's L2 sees one compact spatial
// region whose kept lists overlap, and the rotation spreads chunks that are
// systematically heavier (say, frames with more kept keys) over all XCDs.
// False for padding ids.
__device__ inline bool xcd_item(int bid, int items, int chunk, int64_t* head, int* item) {
  const int x = bid & 7, i = bid >> 3;
  const int h = i / chunk;
  const int it = ((x + h) & 7) * chunk + (i - h * chunk);
  *head = h;
  *item = it;
  return it < items;
}

template <typename OutT>
__device__ inline void store4(OutT* dst, float a, float b, float c, float d);
template <>
__device__ inline void store4<__bf16>(__bf16* dst, float a, float b, float c, float d) {
  bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};   // round to nearest even
  *(bf16x4*)dst = v;
}
template <>
__device__ inline void store4<float>(float* dst, float a, float b, float c, float d) {
  *(f32x4*)dst = f32x4{a, b, c, d};
}

}  // namespace nabla
