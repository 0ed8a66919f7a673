// Measured ceilings of the GPU the library runs on, so that roofline
// fractions can be stated against what this chip sustains as well as against
// its published peaks:
//   * dense bf16 MFMA: every wave issues independent v_mfma_f32_32x32x16_bf16
//     on register operands (four accumulator chains, so the matrix pipe never
//     waits on a result), nothing else in the loop;
//   * HBM streaming: a copy with 16-byte loads and stores, four loads in
//     flight per lane, over buffers far larger than the caches.
// Workgroup 0 also records the core-clock and 100 MHz reference-clock ticks
// around its loop, which gives the clock the chip held while the matrix
// pipes were busy.
#include "hlta_internal.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kChains = 4;

__global__ void __launch_bounds__(kThreads, 2)
mfma_loop_kernel(float* sink, unsigned long long* clocks, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(0.0078125f * float((lane + i) & 15));
    b[i] = static_cast<__bf16>(0.0078125f * float((lane * 3 + i) & 15) - 0.0625f);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  const bool timer = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long t0 = 0, r0 = 0;
  if (timer) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (timer) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (clocks) {
      clocks[0] = t1 - t0;
      clocks[1] = r1 - r0;
    }
  }
  sink[size_t(blockIdx.x) * kThreads + threadIdx.x] = s;
}

// n16 16-byte words, grid-stride; each lane keeps four loads in flight
__global__ void __launch_bounds__(kThreads)
copy_stream_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, long long n16) {
  const long long stride = (long long)gridDim.x * kThreads;
  long long i = (long long)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride], x3 = src[i + 3 * stride];
    dst[i] = x0;
    dst[i + stride] = x1;
    dst[i + 2 * stride] = x2;
    dst[i + 3 * stride] = x3;
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_ceiling_mfma(float* sink, unsigned long long* clocks, int workgroups, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(unsigned(workgroups)), dim3(kThreads), 0, st, sink, clocks, iters);
  return hipGetLastError();
}

hipError_t launch_ceiling_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const long long n16 = (long long)(bytes / 16);
  if (n16 <= 0) return hipSuccess;
  long long blocks = (n16 + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(copy_stream_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace hlta
