// Compressed kept-block lists (lsdiaocha.cn article on NABLA, sec. 5: only the
// compressed sparse matrix is stored instead of the full S x S map).
//
// Per head: row_ptr = exclusive prefix sum of the row counts, col_idx = kept
// block indices of each row in ascending order.  A workgroup handles 64 rows
// of one head: it recomputes the count of all earlier rows of that head (a
// few KB from L2), scans its 64 counts in one wavefront, and then each
// wavefront expands the bit words of its rows with ballot + prefix popcount so
// that consecutive kept blocks are written to consecutive addresses.
#include "nabla_common.hpp"

namespace nabla {

namespace {

constexpr int kRows = 64;

__global__ void __launch_bounds__(256) compact_kernel(const Geo g,
                                                      const uint32_t* __restrict__ bits,
                                                      const int32_t* __restrict__ count,
                                                      int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ col_idx) {
  __shared__ int32_t partial[4];
  __shared__ int32_t starts[kRows];
  const int nb = g.nb;
  const int nw = (nb + 31) >> 5;
  const int64_t head = blockIdx.y;
  const int r0 = blockIdx.x * kRows;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int32_t* cnt = count + head * nb;

  // kept blocks of all rows before r0
  int s = 0;
  for (int i = threadIdx.x; i < r0; i += 256) s += cnt[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) partial[wave] = s;
  __syncthreads();
  const int base = partial[0] + partial[1] + partial[2] + partial[3];

  int32_t* rp = row_ptr + head * (nb + 1);
  if (wave == 0) {
    const int row = r0 + lane;
    const int c = row < nb ? cnt[row] : 0;
    int incl = c;                           // inclusive scan over the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int excl = base + incl - c;
    starts[lane] = excl;
    if (row < nb) rp[row] = excl;
    if (row == nb - 1) rp[nb] = base + incl;
  }
  __syncthreads();

  int32_t* out = col_idx + head * (int64_t)nb * nb;
  const int cap = nb * nb;                  // a row never writes past its head's capacity
  for (int ri = wave; ri < kRows; ri += 4) {
    const int row = r0 + ri;
    if (row >= nb) break;
    const uint32_t* wrow = bits + (head * nb + row) * (int64_t)nw;
    int pos = starts[ri];
    for (int c0 = 0; c0 < nb; c0 += 64) {
      const int c = c0 + lane;
      const bool kept = c < nb && ((wrow[c >> 5] >> (c & 31)) & 1u);
      const uint64_t b = __ballot(kept);
      const int at = pos + __popcll(b & ((1ull << lane) - 1ull));
      if (kept && at >= 0 && at < cap) out[at] = c;
      pos += __popcll(b);
    }
  }
}

}  // namespace

hipError_t launch_compact(const Geo& g, const uint32_t* bits, const int32_t* cnt,
                          int32_t* row_ptr, int32_t* col_idx, hipStream_t s) {
  const dim3 grid((g.nb + kRows - 1) / kRows, (unsigned)g.bh);
  hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, s, g, bits, cnt, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace nabla
