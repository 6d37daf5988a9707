// Achievable rates of this GPU, for reading the kernels' roofline fractions
// against what the chip sustains (the published dense bf16 peak assumes the
// boost clock, the HBM peak the raw interface rate).
//
// * matrix cores: every wavefront issues back-to-back
//   v_mfma_f32_32x32x16_bf16 into four independent accumulators, with no
//   memory traffic in the loop; the grid keeps all 256 CUs full;
// * HBM: a streaming copy, each workgroup on a contiguous chunk, 16-byte
//   non-temporal loads and stores, four in flight per lane.
//
// Built into its own small library, loaded only by the benchmark.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

__global__ void __launch_bounds__(256) mfma_bf16_peak_kernel(int iters, float* __restrict__ out) {
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {        // small operands: the sums stay finite
    a[e] = (__bf16)(1e-3f * (float)((t + e) & 15));
    b[e] = (__bf16)(1e-3f * (float)((t * 3 + e) & 15));
  }
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int i = 0; i < iters; ++i) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r] + acc2[r] + acc3[r];
  out[(size_t)blockIdx.x * 256 + t] = s;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// copy of n 16-byte words: workgroup w streams its own contiguous chunk of
// per words (a multiple of 1024) with non-temporal loads and stores, 4 words
// per lane in flight; the words past grid * per go by a grid-stride loop
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ src,
                                                   u32x4* __restrict__ dst, size_t n) {
  const size_t per = n / gridDim.x / 1024 * 1024;
  const size_t base = (size_t)blockIdx.x * per;
  for (size_t j = threadIdx.x; j < per; j += 1024) {
    const u32x4* s = src + base + j;
    u32x4* d = dst + base + j;
    const u32x4 a = __builtin_nontemporal_load(s), b = __builtin_nontemporal_load(s + 256);
    const u32x4 c = __builtin_nontemporal_load(s + 512), e = __builtin_nontemporal_load(s + 768);
    __builtin_nontemporal_store(a, d);
    __builtin_nontemporal_store(b, d + 256);
    __builtin_nontemporal_store(c, d + 512);
    __builtin_nontemporal_store(e, d + 768);
  }
  for (size_t i = (size_t)gridDim.x * per + (size_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

}  // namespace

extern "C" {

// Launch `grid` workgroups of 256 threads, each wavefront running `iters`
// rounds of 4 matrix instructions; `out` holds grid * 256 floats (device).
// Returns the hipError_t of the launch (0 on success), or -1 for bad sizes.
int nabla_probe_mfma_bf16(int grid, int iters, float* out, hipStream_t stream) {
  if (grid <= 0 || iters <= 0 || out == nullptr) return -1;
  hipLaunchKernelGGL(mfma_bf16_peak_kernel, dim3((unsigned)grid), dim3(256), 0, stream, iters,
                     out);
  return (int)hipGetLastError();
}

// Floating-point operations of one such launch (2 * 32 * 32 * 16 per instruction).
double nabla_probe_mfma_bf16_flops(int grid, int iters) {
  return (double)grid * 4.0 * (double)iters * 4.0 * 2.0 * 32.0 * 32.0 * 16.0;
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned, device
// memory, not overlapping) with `grid` workgroups of 256 threads.  Returns the
// hipError_t of the launch, or -1 for bad arguments.
int nabla_probe_copy(const void* src, void* dst, size_t bytes, int grid, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || grid <= 0 || bytes % 16 != 0 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 16);
  return (int)hipGetLastError();
}

}  // extern "C"
