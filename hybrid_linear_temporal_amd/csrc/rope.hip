// Rotary embedding of the softmax branches' q and k (optional). The pages
// name no positional scheme for the local branches (Kairos abstract, point
// (2), gives them as windows over latent frames); the reading implemented: a
// token's position is (absolute latent frame, row, column) with token p of a
// frame at row p / grid_w, column p % grid_w; coordinate pair i = (x[2i],
// x[2i+1]) is rotated as a complex number by pos_axis * theta^(-j/n), the
// first d/8 pairs following the frame, the next half of the rest the row, the
// others the column (j = index of the pair within its axis, n = pairs of that
// axis). Angles and products in fp32, one rounding to the tensor's dtype.
//
// Bandwidth-bound elementwise pass: a thread rotates 4 consecutive pairs (16
// bytes of bf16, 32 of fp32) of one (token, head) at a time.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;

struct RopeGeom {
  int H, d, P, grid_w;
  float log2_theta;
};

template <typename T>
struct Vec4p;   // 4 coordinate pairs
template <>
struct Vec4p<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int i) const { return static_cast<float>(reinterpret_cast<const bf16*>(&u)[i]); }
  __device__ __forceinline__ void set(int i, float x) { reinterpret_cast<bf16*>(&u)[i] = static_cast<bf16>(x); }
  __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<uint4*>(p) = u; }
};
template <>
struct Vec4p<float> {
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

// cos and sin of the angles of pairs pair0 .. pair0+3 of a token at (frame, p)
__device__ __forceinline__ void angles4(int pair0, long long frame, int p, const RopeGeom& g, float (&c)[4],
                                        float (&s)[4]) {
  const int npairs = g.d / 2, nt = g.d / 8, nh = (npairs - nt) / 2, nw = npairs - nt - nh;
  const float row = float(p / g.grid_w), col = float(p % g.grid_w);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = pair0 + q;
    float pos;
    int j, n;
    if (i < nt) {
      pos = float(frame), j = i, n = nt;
    } else if (i < nt + nh) {
      pos = row, j = i - nt, n = nh;
    } else {
      pos = col, j = i - nt - nh, n = nw;
    }
    const float w = exp2f(-g.log2_theta * float(j) / float(n));
    sincosf(pos * w, &s[q], &c[q]);
  }
}

// Rotate 4 pairs (8 values) by the given angles.
template <typename T>
__device__ __forceinline__ void rotate4(const T* src, T* dst, const float (&c)[4], const float (&s)[4]) {
  Vec4p<T> x;
  x.load(src);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = x.get(2 * q), x1 = x.get(2 * q + 1);
    x.set(2 * q, x0 * c[q] - x1 * s[q]);
    x.set(2 * q + 1, x0 * s[q] + x1 * c[q]);
  }
  x.store(dst);
}

// q, k [B, L, H, d] -> rotated copies; frame of token t of row b =
// frame0(b) + t / P. One workgroup per token (grid-stride): its position is
// wave-uniform, and each thread keeps the angles of one 4-pair group (thread
// index mod d/8) for every head it rotates.
template <typename T>
__global__ void __launch_bounds__(kThreads)
rope_qk_kernel(const T* q, const T* k, T* qr, T* kr, int B, long long L, RopeGeom g, long long f0, int per_rollout,
               RolloutFrames ro) {
  const int groups = g.d / 8;                // 4-pair groups per head vector (a power of two)
  const int grp = threadIdx.x & (groups - 1);
  const int h0 = threadIdx.x / groups, hstep = kThreads / groups;
  for (long long tok = blockIdx.x; tok < (long long)B * L; tok += gridDim.x) {
    const int b = int(tok / L);
    if (skipped(ro.skip, b)) continue;
    const long long t = tok - (long long)b * L;
    const long long frame = (per_rollout ? ro.frame[b] : f0) + t / g.P;
    const int p = int(t % g.P);
    float c[4], sn[4];
    angles4(4 * grp, frame, p, g, c, sn);
    for (int h = h0; h < g.H; h += hstep) {
      const size_t off = (size_t(tok) * g.H + h) * g.d + size_t(grp) * 8;
      rotate4(q + off, qr + off, c, sn);
      rotate4(k + off, kr + off, c, sn);
    }
  }
}

// In place over ring slots: frames first .. first+n-1 of every rollout, frame
// g in slot g mod R of ring [B, R, P, H, d]; one workgroup per token as above.
template <typename T>
__global__ void __launch_bounds__(kThreads)
rope_ring_kernel(T* ring, int B, int R, long long first, int n, RopeGeom g) {
  const int groups = g.d / 8;
  const int grp = threadIdx.x & (groups - 1);
  const int h0 = threadIdx.x / groups, hstep = kThreads / groups;
  const long long tokens = (long long)B * n * g.P;
  for (long long tok = blockIdx.x; tok < tokens; tok += gridDim.x) {
    const int p = int(tok % g.P);
    const long long bf = tok / g.P;
    const int b = int(bf / n);
    const long long frame = first + bf % n;
    const long long slot = frame % R;
    T* base = ring + ((size_t(b) * R + size_t(slot)) * g.P + p) * size_t(g.H) * g.d;
    float c[4], sn[4];
    angles4(4 * grp, frame, p, g, c, sn);
    for (int h = h0; h < g.H; h += hstep) {
      T* x = base + size_t(h) * g.d + size_t(grp) * 8;
      rotate4(x, x, c, sn);
    }
  }
}

unsigned grid_for(long long tokens) {
  return unsigned(tokens < 1 ? 1 : (tokens > (1 << 20) ? (1 << 20) : tokens));
}

}  // namespace

hipError_t launch_rope_qk(const void* q, const void* k, void* qr, void* kr, int B, long long L, int H, int d, int P,
                          int grid_w, float theta, int dt, long long f0, int per_rollout, const RolloutFrames& ro,
                          hipStream_t st) {
  if (B <= 0 || L <= 0) return hipSuccess;
  const RopeGeom g{H, d, P, grid_w, log2f(theta)};
  const unsigned grid = grid_for((long long)B * L);
  if (dt == HLTA_BF16)
    hipLaunchKernelGGL(rope_qk_kernel<bf16>, dim3(grid), dim3(kThreads), 0, st, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(k), static_cast<bf16*>(qr), static_cast<bf16*>(kr), B, L, g, f0,
                       per_rollout, ro);
  else
    hipLaunchKernelGGL(rope_qk_kernel<float>, dim3(grid), dim3(kThreads), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<float*>(qr), static_cast<float*>(kr), B, L, g, f0,
                       per_rollout, ro);
  return hipGetLastError();
}

hipError_t launch_rope_ring(void* ring, int B, int R, long long first, int n, int H, int d, int P, int grid_w,
                            float theta, int dt, hipStream_t st) {
  if (B <= 0 || n <= 0) return hipSuccess;
  const RopeGeom g{H, d, P, grid_w, log2f(theta)};
  const unsigned grid = grid_for((long long)B * n * P);
  if (dt == HLTA_BF16)
    hipLaunchKernelGGL(rope_ring_kernel<bf16>, dim3(grid), dim3(kThreads), 0, st, static_cast<bf16*>(ring), B, R,
                       first, n, g);
  else
    hipLaunchKernelGGL(rope_ring_kernel<float>, dim3(grid), dim3(kThreads), 0, st, static_cast<float*>(ring), B, R,
                       first, n, g);
  return hipGetLastError();
}

}  // namespace hlta
