// Generic SWA + DSWA softmax-attention kernel (fp32 arithmetic, any d in
// {32, 64, 128}, float32 or bf16 inputs).
//
// Exact attention over every legal (query, key) pair, computed tile by tile
// with a running max and sum so the score matrix never leaves the chip
// (long-context page, section 03 on FlashAttention). Frame sets per query
// frame f: SWA frames f-W+1 .. f, DSWA frames f - dil*r, r = 1..taps (Kairos
// abstract, point (2)); keys of the listed frames form one virtual sequence
// per branch.
//
// One workgroup = 64 query rows of one frame, one head, one batch row;
// 4 threads per row, each owning d/4 output columns.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kRows = 64;      // query rows per workgroup
constexpr int kThreads = 256;  // 4 threads per row
constexpr int kKeys = 32;      // keys per LDS tile

template <typename Tin, typename Tout, int D>
__global__ void __launch_bounds__(kThreads)
attn_generic_kernel(AttnParams p) {
  constexpr int DP = D / 4;  // columns per thread
  __shared__ float Ks[kKeys][D + 1];
  __shared__ float Vs[kKeys][D + 1];

  const int tiles_per_frame = (p.P + kRows - 1) / kRows;
  const int fq = blockIdx.x / tiles_per_frame;             // query frame within the call
  const int row0 = (blockIdx.x % tiles_per_frame) * kRows;
  const int h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.ro.skip, b)) return;
  const int tid = threadIdx.x;
  const int r = tid >> 2, c = tid & 3;
  const int prow = row0 + r;                               // token inside the frame
  const bool row_ok = prow < p.P;
  const long long f = call_frame(p, b) + fq;               // absolute frame

  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* kmain = static_cast<const Tin*>(p.k);
  const Tin* vmain = static_cast<const Tin*>(p.v);
  const Tin* kring = static_cast<const Tin*>(p.ring_k);
  const Tin* vring = static_cast<const Tin*>(p.ring_v);
  const size_t tok_stride = size_t(p.H) * D;
  const size_t qoff = ((size_t(b) * p.T * p.P + size_t(fq) * p.P + prow) * p.H + h) * D + c * DP;

  float qr[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) qr[i] = row_ok ? to_f32(q[qoff + i]) * p.scale_log2 : 0.f;

  const int nswa = swa_count(f, p.W);
  const int ndswa = dswa_count(f, p.dil, p.taps);

  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    float m = -INFINITY, l = 0.f;
    float acc[DP];
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] = 0.f;

    for (long long t0 = 0; t0 < nk; t0 += kKeys) {
      __syncthreads();
      for (int e = tid; e < kKeys * D; e += kThreads) {
        const int jj = e / D, col = e % D;
        const long long j = t0 + jj;
        float kv = 0.f, vv = 0.f;
        if (j < nk) {
          const int s = int(j / p.P), pk = int(j % p.P);
          const long long g = branch_frame(branch, f, nswa, p.dil, s);
          const size_t off = size_t(pk) * tok_stride + col;
          kv = to_f32(key_frame_ptr<Tin, D>(kmain, kring, p, b, h, g)[off]);
          vv = to_f32(key_frame_ptr<Tin, D>(vmain, vring, p, b, h, g)[off]);
        }
        Ks[jj][col] = kv;
        Vs[jj][col] = vv;
      }
      __syncthreads();

      float s[kKeys];
      float tmax = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kKeys; ++jj) {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < DP; ++i) part += qr[i] * Ks[jj][c * DP + i];
        part += __shfl_xor(part, 1, 4);
        part += __shfl_xor(part, 2, 4);
        s[jj] = (t0 + jj < nk) ? part : -INFINITY;
        tmax = fmaxf(tmax, s[jj]);
      }
      const float mnew = fmaxf(m, tmax);
      const float corr = exp2f(m - mnew);
      l *= corr;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] *= corr;
#pragma unroll
      for (int jj = 0; jj < kKeys; ++jj) {
        const float pj = exp2f(s[jj] - mnew);
        l += pj;
#pragma unroll
        for (int i = 0; i < DP; ++i) acc[i] += pj * Vs[jj][c * DP + i];
      }
      m = mnew;
    }

    const float inv = l > 0.f ? 1.f / l : 0.f;
    Tout* out = static_cast<Tout*>(branch == 0 ? p.o_swa : p.o_dswa);
    if (p.R == 0 && p.lse && row_ok && c == 0)
      p.lse[((size_t(branch) * p.B + b) * p.H + h) * (size_t(p.T) * p.P) + size_t(fq) * p.P + prow] =
          nk > 0 ? m + log2f(l) : 0.f;
    if (row_ok) {
#pragma unroll
      for (int i = 0; i < DP; ++i) out[qoff + i] = from_f32<Tout>(acc[i] * inv);
    }
  }
}

template <typename Tin, typename Tout, int D>
hipError_t launch_t(const AttnParams& p, hipStream_t st) {
  const int tiles = (p.P + kRows - 1) / kRows;
  dim3 grid(unsigned(p.T) * tiles, p.H, p.B);
  hipLaunchKernelGGL((attn_generic_kernel<Tin, Tout, D>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_generic(const AttnParams& p, int d, int in_dt, int out_dt, hipStream_t st) {
  if (in_dt == HLTA_F32) {
    if (d == 32) return launch_t<float, float, 32>(p, st);
    if (d == 64) return launch_t<float, float, 64>(p, st);
    return launch_t<float, float, 128>(p, st);
  }
  if (out_dt == HLTA_BF16) {
    if (d == 32) return launch_t<bf16, bf16, 32>(p, st);
    if (d == 64) return launch_t<bf16, bf16, 64>(p, st);
    return launch_t<bf16, bf16, 128>(p, st);
  }
  if (d == 32) return launch_t<bf16, float, 32>(p, st);
  if (d == 64) return launch_t<bf16, float, 64>(p, st);
  return launch_t<bf16, float, 128>(p, st);
}

}  // namespace hlta
