// Input quantisation of the FP8 (e4m3) variant of the softmax branches: q, k,
// v [B, L, H, d] -> e4m3 codes with one float32 scale per (batch row, head,
// tensor), s = max|x| / 448 (1 for an all-zero head); code = e4m3(x / s), x / s
// in float32 clamped to +-448, rounded to nearest (ties to even) by the
// hardware conversion. The pages mention low-precision attention without a
// method; this per-head scaling is the reading implemented.
//
// Three bandwidth-bound passes on the caller's stream: clear the maxima, take
// max|x| per (b, h, tensor) (block maxima merged with atomicMax on the
// non-negative float bit patterns, which order like the floats), then convert
// (every element read once more) and turn the maxima into scales in place.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;
constexpr float kE4m3Max = 448.f;
constexpr int kTokensPerBlock = 512;

__global__ void __launch_bounds__(kThreads) clear_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// max |x| over the elements of one 16-byte chunk
__device__ __forceinline__ float chunk_absmax(const bf16*, const uint4& u) {
  const bf16* e = reinterpret_cast<const bf16*>(&u);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(static_cast<float>(e[i])));
  return m;
}
__device__ __forceinline__ float chunk_absmax(const float*, const uint4& u) {
  const float* e = reinterpret_cast<const float*>(&u);
  return fmaxf(fmaxf(fabsf(e[0]), fabsf(e[1])), fmaxf(fabsf(e[2]), fabsf(e[3])));
}

// grid: (ceil(L / kTokensPerBlock), H, B * 3); one 16-byte chunk per thread,
// cpr chunks per token row of one head (d * sizeof(T) / 16), 256 / cpr rows at a time.
template <typename T>
__global__ void __launch_bounds__(kThreads)
absmax_kernel(const T* q, const T* k, const T* v, unsigned* amax, long long L, int H, int d) {
  const int h = blockIdx.y, b = blockIdx.z / 3, t = blockIdx.z % 3;
  const T* x = t == 0 ? q : (t == 1 ? k : v);
  const int cpr = int(d * sizeof(T) / 16);
  const int rows = kThreads / cpr;
  const int chunk = threadIdx.x % cpr;
  const long long t0 = (long long)blockIdx.x * kTokensPerBlock;
  const long long t1 = t0 + kTokensPerBlock < L ? t0 + kTokensPerBlock : L;
  float m = 0.f;
  for (long long tok = t0 + threadIdx.x / cpr; tok < t1; tok += rows) {
    const uint4 u = reinterpret_cast<const uint4*>(x + ((size_t(b) * L + size_t(tok)) * H + h) * d)[chunk];
    m = fmaxf(m, chunk_absmax(x, u));
  }
  // wave maximum, then the block's through LDS
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float bm = wm[0];
    for (int w = 1; w < kThreads / 64; ++w) bm = fmaxf(bm, wm[w]);
    atomicMax(amax + (size_t(b) * H + h) * 3 + t, __float_as_uint(bm));
  }
}

__device__ __forceinline__ float scale_of(unsigned amax_bits) {
  const float a = __uint_as_float(amax_bits);
  return a > 0.f ? a / kE4m3Max : 1.f;
}

template <typename T>
struct Load8;
template <>
struct Load8<bf16> {
  static __device__ __forceinline__ void get(const bf16* p, float (&f)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const bf16* e = reinterpret_cast<const bf16*>(&u);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = static_cast<float>(e[i]);
  }
};
template <>
struct Load8<float> {
  static __device__ __forceinline__ void get(const float* p, float (&f)[8]) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], c = reinterpret_cast<const uint4*>(p)[1];
    const float* x = reinterpret_cast<const float*>(&a);
    const float* y = reinterpret_cast<const float*>(&c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = x[i];
      f[4 + i] = y[i];
    }
  }
};

// one workgroup per token (grid-stride): its batch row is wave-uniform; a
// thread converts 8 consecutive values of one (tensor, head) at a time
template <typename T>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const T* q, const T* k, const T* v, unsigned char* q8, unsigned char* k8, unsigned char* v8,
                const unsigned* amax, int B, long long L, int H, int d) {
  const int d8 = d / 8, per_tensor = H * d8;
  for (long long tok = blockIdx.x; tok < (long long)B * L; tok += gridDim.x) {
    const int b = int(tok / L);
    for (int i = threadIdx.x; i < 3 * per_tensor; i += kThreads) {
      const int t = i / per_tensor, r = i - t * per_tensor, h = r / d8;
      const float s = scale_of(amax[(size_t(b) * H + h) * 3 + t]);
      const size_t o = size_t(tok) * per_tensor * 8 + size_t(r) * 8;
      const T* x = (t == 0 ? q : (t == 1 ? k : v)) + o;
      unsigned char* y = (t == 0 ? q8 : (t == 1 ? k8 : v8)) + o;
      float f[8];
      Load8<T>::get(x, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fminf(fmaxf(f[e] / s, -kE4m3Max), kE4m3Max);
      int lo = 0, hi = 0;
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], lo, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], hi, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
      *reinterpret_cast<uint2*>(y) = make_uint2(unsigned(lo), unsigned(hi));
    }
  }
}

__global__ void __launch_bounds__(kThreads) finalize_kernel(unsigned* amax_to_scale, int n) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < n) amax_to_scale[i] = __float_as_uint(scale_of(amax_to_scale[i]));
}

}  // namespace

hipError_t launch_quantize_e4m3(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
                                float* scales, int B, long long L, int H, int d, int dt, hipStream_t st) {
  const int ns = B * H * 3;
  unsigned* amax = reinterpret_cast<unsigned*>(scales);
  hipLaunchKernelGGL(clear_kernel, dim3((ns + kThreads - 1) / kThreads), dim3(kThreads), 0, st, amax, ns);
  if (L > 0) {
    const dim3 grid(unsigned((L + kTokensPerBlock - 1) / kTokensPerBlock), unsigned(H), unsigned(B * 3));
    long long blocks = (long long)B * L;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    if (dt == HLTA_BF16) {
      hipLaunchKernelGGL(absmax_kernel<bf16>, grid, dim3(kThreads), 0, st, static_cast<const bf16*>(q),
                         static_cast<const bf16*>(k), static_cast<const bf16*>(v), amax, L, H, d);
      hipLaunchKernelGGL(quantize_kernel<bf16>, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
                         static_cast<unsigned char*>(q8), static_cast<unsigned char*>(k8),
                         static_cast<unsigned char*>(v8), amax, B, L, H, d);
    } else {
      hipLaunchKernelGGL(absmax_kernel<float>, grid, dim3(kThreads), 0, st, static_cast<const float*>(q),
                         static_cast<const float*>(k), static_cast<const float*>(v), amax, L, H, d);
      hipLaunchKernelGGL(quantize_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                         static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                         static_cast<unsigned char*>(q8), static_cast<unsigned char*>(k8),
                         static_cast<unsigned char*>(v8), amax, B, L, H, d);
    }
  }
  hipLaunchKernelGGL(finalize_kernel, dim3((ns + kThreads - 1) / kThreads), dim3(kThreads), 0, st, amax, ns);
  return hipGetLastError();
}

}  // namespace hlta
