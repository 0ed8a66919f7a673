// Ring-buffer copies of the streaming path: frame g of every rollout goes to
// ring slot g mod R, so a step finds the K/V of past frames without the clip
// being recomputed (Kairos article on zhichai.net, section 2.3, streaming
// tokens).
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

}  // namespace

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
