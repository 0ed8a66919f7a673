// Elementwise kernels around the branches: the per-head mix of the three
// branch outputs, and the ring-buffer copies of the streaming path (frame g
// of every rollout goes to ring slot g mod R, so a step finds the K/V of past
// frames without the clip being recomputed; Kairos article on zhichai.net,
// section 2.3, streaming tokens).
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;

// grid: (ceil(frame_vec / kThreads / kPerThread), n_frames, B); 16-byte vectors
__global__ void __launch_bounds__(kThreads)
ring_store_kernel(const uint4* src, long long src_frames, long long src_f0, uint4* ring, int R,
                  long long first_frame, long long frame_vec) {
  const long long g = first_frame + blockIdx.y;
  const int b = blockIdx.z;
  const long long slot = g % R;
  const uint4* s = src + (size_t(b) * src_frames + size_t(g - src_f0)) * frame_vec;
  uint4* d = ring + (size_t(b) * R + size_t(slot)) * frame_vec;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < frame_vec;
       i += (long long)gridDim.x * kThreads)
    d[i] = s[i];
}

// One frame per rollout, each into the slot of its own frame: rollout b's
// frame (src row b) goes to ring slot frame[b] mod R; rollouts in skip are
// left alone. grid: (blocks, 1, B).
__global__ void __launch_bounds__(kThreads)
ring_store_rollouts_kernel(const uint4* src, uint4* ring, int R, long long frame_vec, RolloutFrames sel) {
  const int b = blockIdx.z;
  if (skipped(sel.skip, b)) return;
  const long long slot = sel.frame[b] % R;
  const uint4* s = src + size_t(b) * frame_vec;
  uint4* d = ring + (size_t(b) * R + size_t(slot)) * frame_vec;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < frame_vec;
       i += (long long)gridDim.x * kThreads)
    d[i] = s[i];
}

// o_mix = w[h][0] o_swa + w[h][1] o_dswa + w[h][2] o_gdn, elementwise over the
// stored branch outputs (Kairos abstract, point (2): the three branches are
// mixed per head), with one fp32 rounding order for every caller:
// fma(w2, gdn, fma(w1, dswa, w0 * swa)), then one rounding to the output type.
// One thread per 8 consecutive values of one (token, head); 16-byte vectors,
// loaded and stored non-temporally since the mix streams each value once
// (bf16: 0.221 -> 0.205 ms per 480P call against plain ones, same results).
typedef unsigned v4u __attribute__((ext_vector_type(4)));
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) {
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    u = make_uint4(x[0], x[1], x[2], x[3]);
  }
  __device__ __forceinline__ float get(int i) const {
    const bf16* e = reinterpret_cast<const bf16*>(&u);
    return static_cast<float>(e[i]);
  }
  __device__ __forceinline__ void set(int i, float x) { reinterpret_cast<bf16*>(&u)[i] = static_cast<bf16>(x); }
  __device__ __forceinline__ void store(bf16* p) const {
    __builtin_nontemporal_store(v4u{u.x, u.y, u.z, u.w}, reinterpret_cast<v4u*>(p));
  }
};
template <>
struct Vec8<float> {
  uint4 u[2];
  __device__ __forceinline__ void load(const float* p) {
    u[0] = reinterpret_cast<const uint4*>(p)[0];
    u[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ float get(int i) const { return reinterpret_cast<const float*>(u)[i]; }
  __device__ __forceinline__ void set(int i, float x) { reinterpret_cast<float*>(u)[i] = x; }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<uint4*>(p)[0] = u[0];
    reinterpret_cast<uint4*>(p)[1] = u[1];
  }
};

template <typename T>
__global__ void __launch_bounds__(kThreads)
mix_kernel(const T* swa, const T* dswa, const T* gdn, T* mix, const float* w, long long n8, int H, int d8,
           unsigned long long skip, long long row8) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n8; i += (long long)gridDim.x * kThreads) {
    if (skip != 0 && skipped(skip, int(i / row8))) continue;   // rollout left out: its rows stay as they are
    const int h = int((i / d8) % H);
    const float w0 = w[3 * h], w1 = w[3 * h + 1], w2 = w[3 * h + 2];
    Vec8<T> a, b, g, o;
    a.load(swa + 8 * i);
    b.load(dswa + 8 * i);
    g.load(gdn + 8 * i);
#pragma unroll
    for (int e = 0; e < 8; ++e) o.set(e, fmaf(w2, g.get(e), fmaf(w1, b.get(e), w0 * a.get(e))));
    o.store(mix + 8 * i);
  }
}

// dst = src, or dst = 0 when src is null, over n 4-byte words (grid-stride).
// A kernel rather than hipMemcpyAsync / hipMemsetAsync, so that every entry
// point records only kernel nodes when a caller captures it in a HIP graph.
__global__ void __launch_bounds__(kThreads)
copy_words_kernel(unsigned* dst, const unsigned* src, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads)
    dst[i] = src ? src[i] : 0u;
}

}  // namespace

hipError_t launch_copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t st) {
  const long long n = (long long)(bytes / 4);
  if (n <= 0) return hipSuccess;
  long long blocks = (n + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(copy_words_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, st, static_cast<unsigned*>(dst),
                     static_cast<const unsigned*>(src), n);
  return hipGetLastError();
}

hipError_t launch_mix(const void* o_swa, const void* o_dswa, const void* o_gdn, void* o_mix, const float* mix_w,
                      long long ntok, int H, int d, int out_dt, hipStream_t st, unsigned long long skip,
                      long long rollout_tokens) {
  const long long n8 = ntok * H * (d / 8);
  const long long row8 = rollout_tokens * H * (d / 8);
  if (n8 <= 0) return hipSuccess;
  long long blocks = (n8 + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (out_dt == HLTA_BF16)
    hipLaunchKernelGGL(mix_kernel<bf16>, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                       static_cast<const bf16*>(o_swa), static_cast<const bf16*>(o_dswa),
                       static_cast<const bf16*>(o_gdn), static_cast<bf16*>(o_mix), mix_w, n8, H, d / 8, skip, row8);
  else
    hipLaunchKernelGGL(mix_kernel<float>, dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                       static_cast<const float*>(o_swa), static_cast<const float*>(o_dswa),
                       static_cast<const float*>(o_gdn), static_cast<float*>(o_mix), mix_w, n8, H, d / 8, skip, row8);
  return hipGetLastError();
}

hipError_t launch_ring_store_rollouts(const void* src, void* ring, int R, int B, long long frame_elems, int elem,
                                     const RolloutFrames& sel, hipStream_t st) {
  const long long frame_vec = frame_elems * elem / 16;   // frame bytes are a multiple of 16 (d >= 32)
  long long blocks = (frame_vec + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(ring_store_rollouts_kernel, dim3(unsigned(blocks), 1, B), dim3(kThreads), 0, st,
                     static_cast<const uint4*>(src), static_cast<uint4*>(ring), R, frame_vec, sel);
  return hipGetLastError();
}

hipError_t launch_ring_store(const void* src, long long src_frames, long long src_f0, void* ring, int R,
                             long long first_frame, long long n_frames, int B, long long frame_elems,
                             int elem, hipStream_t st) {
  if (n_frames <= 0) return hipSuccess;
  const long long frame_vec = frame_elems * elem / 16;   // frame bytes are a multiple of 16 (d >= 32)
  long long blocks = (frame_vec + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(ring_store_kernel, dim3(unsigned(blocks), unsigned(n_frames), B), dim3(kThreads), 0, st,
                     static_cast<const uint4*>(src), src_frames, src_f0, static_cast<uint4*>(ring), R,
                     first_frame, frame_vec);
  return hipGetLastError();
}

}  // namespace hlta
