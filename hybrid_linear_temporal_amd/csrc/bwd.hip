// Backward of the operator (gradients for training): given dL/do_mix, the
// gradients of q, k, v, the gates, the mix weights and the start state. The
// branch gradients are do_i = w[h, i] * d_mix (the mix is linear). Kernels
// for any supported d and input dtype, accumulating in fp32:
//
//  * softmax branches (exact attention, so its gradient is the textbook one;
//    long-context page, section 03 on tiled exact attention): a recompute pass
//    stores per query row the log2-sum-exp and D = do . o; a query-major pass
//    accumulates dq = s sum_k P (do . v_k - D) k; a key-major pass walks, for
//    each key frame, the query frames whose frame set holds it and
//    accumulates dv = sum_i P do_i and dk = s sum_i P (do_i . v - D_i) q_i;
//  * gated delta rule (Kairos related-work page, row A; long-context page,
//    section 06): per chunk of C tokens, in parallel, the chunk's affine map
//    S_end = S_start A_c + U_c and its own adjoint from zero X_c (matrix form,
//    gdn_bwd_mat.hip); then two short chains over chunks give every chunk's
//    start state and the adjoint reaching its end; then, per chunk in
//    parallel again, the token gradients in matrix form (all in
//    gdn_bwd_mat.hip).
//    The chunk products there run on bf16 MFMA with each fp32 operand split
//    into a bf16 head and a bf16 remainder (three products), which keeps
//    them close to fp32 accuracy;
//  * mix weights: dw[h, i] = <d_mix, o_i> over the stored branch outputs.
// With bf16 inputs and outputs, d = 128 and P >= 64 the softmax branches run
// on the bf16 MFMA kernels of attn_bwd_mfma.hip instead.
#include <type_traits>

#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ float ld(const T* p, size_t i) {
  return static_cast<float>(p[i]);
}

// ---------------------------------------------------------------------------
// softmax branches
// ---------------------------------------------------------------------------

constexpr int kRows = 64;   // query (or key) rows per workgroup, 4 threads per row
constexpr int kTile = 32;   // rows of the other side staged in LDS at a time

// sum over the 4 threads of a row (lanes 4r .. 4r+3)
__device__ __forceinline__ float row4(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Recompute pass: lse2 (log2 of the softmax denominator, scores in log2 units)
// and D = do . o of every query row, per branch. grid (tiles of the frame * T, H, B)
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kThreads)
attn_bwd_stats(AttnParams p, const Tg* d_mix, const float* mix_w, float* lse2, float* dsum) {
  constexpr int DP = D / 4;
  __shared__ float Ks[kTile][D + 1], Vs[kTile][D + 1];
  const int tiles = (p.P + kRows - 1) / kRows;
  const int fq = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * kRows;
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, r = tid >> 2, c = tid & 3;
  const int prow = row0 + r;
  const bool ok = prow < p.P;
  const long long f = fq;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const size_t tok = size_t(b) * p.T * p.P + size_t(fq) * p.P + prow;
  float qr[DP], g[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qr[i] = ok ? ld(q, tok * HD + h * D + c * DP + i) * p.scale_log2 : 0.f;
    g[i] = ok ? ld(d_mix, tok * HD + h * D + c * DP + i) : 0.f;
  }
  const int nswa = swa_count(f, p.W), ndswa = dswa_count(f, p.dil, p.taps);
  for (int branch = 0; branch < 2; ++branch) {
    const int nfr = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nfr * p.P;
    float m = -INFINITY, l = 0.f, acc[DP];
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] = 0.f;
    for (long long t0 = 0; t0 < nk; t0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * D; e += kThreads) {
        const int jj = e / D, col = e % D;
        const long long j = t0 + jj;
        float kv = 0.f, vv = 0.f;
        if (j < nk) {
          const long long gfr = branch_frame(branch, f, nswa, p.dil, int(j / p.P));
          const size_t kt = (size_t(b) * p.T * p.P + size_t(gfr) * p.P + size_t(j % p.P)) * HD + h * D + col;
          kv = ld(k, kt);
          vv = ld(v, kt);
        }
        Ks[jj][col] = kv;
        Vs[jj][col] = vv;
      }
      __syncthreads();
      const int nj = int(nk - t0 < kTile ? nk - t0 : kTile);
      for (int jj = 0; jj < nj; ++jj) {
        float sc = 0.f;
#pragma unroll
        for (int i = 0; i < DP; ++i) sc += qr[i] * Ks[jj][c * DP + i];
        sc = row4(sc);
        const float mn = fmaxf(m, sc);
        const float al = exp2f(m - mn), e = exp2f(sc - mn);
        l = l * al + e;
#pragma unroll
        for (int i = 0; i < DP; ++i) acc[i] = acc[i] * al + e * Vs[jj][c * DP + i];
        m = mn;
      }
    }
    float dd = 0.f;
    if (nk > 0) {
#pragma unroll
      for (int i = 0; i < DP; ++i) dd += g[i] * acc[i];
      dd = row4(dd) / l;
    }
    if (ok && c == 0) {
      const size_t o = (size_t(branch) * p.B * p.T * p.P + tok) * p.H + h;
      lse2[o] = nk > 0 ? m + log2f(l) : 0.f;
      dsum[o] = dd * mix_w[3 * h + branch];   // D of do = w * d_mix
    }
  }
}

// dq, query-major: dq += s * sum_k P (do . v_k - D) k over both branches
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kThreads)
attn_bwd_dq(AttnParams p, const Tg* d_mix, const float* mix_w, const float* lse2, const float* dsum, float* dq,
            float scale) {
  constexpr int DP = D / 4;
  __shared__ float Ks[kTile][D + 1], Vs[kTile][D + 1];
  const int tiles = (p.P + kRows - 1) / kRows;
  const int fq = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * kRows;
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, r = tid >> 2, c = tid & 3;
  const int prow = row0 + r;
  const bool ok = prow < p.P;
  const long long f = fq;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const size_t tok = size_t(b) * p.T * p.P + size_t(fq) * p.P + prow;
  float qr[DP], g[DP], dqa[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    qr[i] = ok ? ld(q, tok * HD + h * D + c * DP + i) * p.scale_log2 : 0.f;
    g[i] = ok ? ld(d_mix, tok * HD + h * D + c * DP + i) : 0.f;
    dqa[i] = 0.f;
  }
  const int nswa = swa_count(f, p.W), ndswa = dswa_count(f, p.dil, p.taps);
  for (int branch = 0; branch < 2; ++branch) {
    const int nfr = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nfr * p.P;
    const float w = mix_w[3 * h + branch];
    const size_t so = (size_t(branch) * p.B * p.T * p.P + (ok ? tok : 0)) * p.H + h;
    const float L2 = lse2[so], Dd = dsum[so];
    for (long long t0 = 0; t0 < nk; t0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * D; e += kThreads) {
        const int jj = e / D, col = e % D;
        const long long j = t0 + jj;
        float kv = 0.f, vv = 0.f;
        if (j < nk) {
          const long long gfr = branch_frame(branch, f, nswa, p.dil, int(j / p.P));
          const size_t kt = (size_t(b) * p.T * p.P + size_t(gfr) * p.P + size_t(j % p.P)) * HD + h * D + col;
          kv = ld(k, kt);
          vv = ld(v, kt);
        }
        Ks[jj][col] = kv;
        Vs[jj][col] = vv;
      }
      __syncthreads();
      const int nj = int(nk - t0 < kTile ? nk - t0 : kTile);
      for (int jj = 0; jj < nj; ++jj) {
        float sc = 0.f, dp = 0.f;
#pragma unroll
        for (int i = 0; i < DP; ++i) {
          sc += qr[i] * Ks[jj][c * DP + i];
          dp += g[i] * Vs[jj][c * DP + i];
        }
        sc = row4(sc);
        dp = row4(dp) * w;
        const float pr = exp2f(sc - L2);
        const float ds = pr * (dp - Dd);
#pragma unroll
        for (int i = 0; i < DP; ++i) dqa[i] += ds * Ks[jj][c * DP + i];
      }
    }
  }
  if (ok) {
#pragma unroll
    for (int i = 0; i < DP; ++i) dq[tok * HD + h * D + c * DP + i] = scale * dqa[i];
  }
}

// dk, dv, key-major: rows of this workgroup are keys of frame g; the queries
// that read them are those of frames f with g in their frame set
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kThreads)
attn_bwd_dkdv(AttnParams p, const Tg* d_mix, const float* mix_w, const float* lse2, const float* dsum, float* dk,
              float* dv, float scale) {
  constexpr int DP = D / 4;
  __shared__ float Qs[kTile][D + 1], Gs[kTile][D + 1];
  __shared__ float Ls[kTile], Ds[kTile];
  const int tiles = (p.P + kRows - 1) / kRows;
  const int gk = blockIdx.x / tiles, row0 = (blockIdx.x % tiles) * kRows;
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x, r = tid >> 2, c = tid & 3;
  const int krow = row0 + r;
  const bool ok = krow < p.P;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const size_t ktok = size_t(b) * p.T * p.P + size_t(gk) * p.P + krow;
  float kr[DP], vr[DP], dka[DP], dva[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    kr[i] = ok ? ld(k, ktok * HD + h * D + c * DP + i) * p.scale_log2 : 0.f;
    vr[i] = ok ? ld(v, ktok * HD + h * D + c * DP + i) : 0.f;
    dka[i] = dva[i] = 0.f;
  }
  for (int branch = 0; branch < 2; ++branch) {
    const float w = mix_w[3 * h + branch];
    // query frames whose branch frame set holds frame gk
    const int nq = branch == 0 ? p.W : p.taps;
    for (int qi = 0; qi < nq; ++qi) {
      const long long f = branch == 0 ? (long long)gk + qi : (long long)gk + (long long)p.dil * (qi + 1);
      if (f >= p.T) break;
      for (int t0 = 0; t0 < p.P; t0 += kTile) {
        __syncthreads();
        for (int e = tid; e < kTile * D; e += kThreads) {
          const int ii = e / D, col = e % D;
          const int i = t0 + ii;
          float qv = 0.f, gv = 0.f;
          if (i < p.P) {
            const size_t qt = (size_t(b) * p.T * p.P + size_t(f) * p.P + i) * HD + h * D + col;
            qv = ld(q, qt);
            gv = ld(d_mix, qt) * w;
          }
          Qs[ii][col] = qv;
          Gs[ii][col] = gv;
        }
        if (tid < kTile) {
          const int i = t0 + tid;
          float L2 = 0.f, Dd = 0.f;
          if (i < p.P) {
            const size_t so = (size_t(branch) * p.B * p.T * p.P + size_t(b) * p.T * p.P + size_t(f) * p.P + i) * p.H + h;
            L2 = lse2[so];
            Dd = dsum[so];
          }
          Ls[tid] = L2;
          Ds[tid] = Dd;
        }
        __syncthreads();
        const int ni = p.P - t0 < kTile ? p.P - t0 : kTile;
        for (int ii = 0; ii < ni; ++ii) {
          float sc = 0.f, dp = 0.f;
#pragma unroll
          for (int i = 0; i < DP; ++i) {
            sc += kr[i] * Qs[ii][c * DP + i];
            dp += vr[i] * Gs[ii][c * DP + i];
          }
          sc = row4(sc);
          dp = row4(dp);
          const float pr = exp2f(sc - Ls[ii]);
          const float ds = pr * (dp - Ds[ii]);
#pragma unroll
          for (int i = 0; i < DP; ++i) {
            dva[i] += pr * Gs[ii][c * DP + i];
            dka[i] += ds * Qs[ii][c * DP + i];
          }
        }
      }
    }
  }
  if (ok) {
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      dk[ktok * HD + h * D + c * DP + i] = scale * dka[i];
      dv[ktok * HD + h * D + c * DP + i] = dva[i];
    }
  }
}

// ---------------------------------------------------------------------------
// gated delta rule
// ---------------------------------------------------------------------------

// dw[h, i] = <d_mix, o_i> in two deterministic stages: per-head partial sums
// over grid.y slices (grid (H, slices)), then their sum in a fixed order.
template <typename Tg, typename Tout>
__global__ void __launch_bounds__(kThreads)
dmix_partial(const Tg* d_mix, const Tout* o_swa, const Tout* o_dswa, const Tout* o_gdn, float* part, long long ntok,
             int H, int d) {
  const int h = blockIdx.x;
  float s[3] = {0.f, 0.f, 0.f};
  for (long long e = (long long)blockIdx.y * kThreads + threadIdx.x; e < ntok * d;
       e += (long long)gridDim.y * kThreads) {
    const size_t i = size_t(e / d) * H * d + size_t(h) * d + size_t(e % d);
    const float g = ld(d_mix, i);
    s[0] += g * ld(o_swa, i);
    s[1] += g * ld(o_dswa, i);
    s[2] += g * ld(o_gdn, i);
  }
  __shared__ float red[3][kThreads / 64];
  for (int j = 0; j < 3; ++j) {
    float x = s[j];
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((threadIdx.x & 63) == 0) red[j][threadIdx.x >> 6] = x;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    float x = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) x += red[threadIdx.x][w];
    part[(size_t(h) * gridDim.y + blockIdx.y) * 3 + threadIdx.x] = x;
  }
}

__global__ void __launch_bounds__(64) dmix_final(const float* part, float* dw, int H, int nblk) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= 3 * H) return;
  const int h = i / 3, j = i % 3;
  float x = 0.f;
  for (int k = 0; k < nblk; ++k) x += part[(size_t(h) * nblk + k) * 3 + j];
  dw[i] = x;
}

template <typename Tin, typename Tg, int D>
hipError_t launch_bwd_t(const BwdArgs& x, hipStream_t st) {
  const AttnParams& p = x.attn;
  const int tiles = (p.P + kRows - 1) / kRows;
  const dim3 grid(unsigned(tiles * p.T), unsigned(p.H), unsigned(p.B));
  const Tg* g = static_cast<const Tg*>(x.d_mix);
  if (x.attn_mfma) {
    const hipError_t e = launch_attn_bwd_mfma(p, x.d_mix, x.o_swa, x.o_dswa, x.mix_w, x.lse2, x.lse_given != 0,
                                              x.dsum, x.dq, x.dk, x.dv, x.scale, st);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((attn_bwd_stats<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum);
    hipLaunchKernelGGL((attn_bwd_dq<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum,
                       x.dq, x.scale);
    hipLaunchKernelGGL((attn_bwd_dkdv<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum,
                       x.dk, x.dv, x.scale);
  }
  const int in_dt = std::is_same<Tin, bf16>::value ? HLTA_BF16 : HLTA_F32;
  const int out_dt = std::is_same<Tg, bf16>::value ? HLTA_BF16 : HLTA_F32;
  hipError_t e = launch_gdn_bwd_mat(x, D, in_dt, out_dt, 0, st);
  if (e != hipSuccess) return e;
  e = launch_gdn_bwd_mat(x, D, in_dt, out_dt, 2, st);
  if (e != hipSuccess) return e;
  return launch_gdn_bwd_mat(x, D, in_dt, out_dt, 1, st);
}

template <typename Tin, typename Tg>
hipError_t launch_bwd_d(const BwdArgs& x, int d, hipStream_t st) {
  switch (d) {
    case 32: return launch_bwd_t<Tin, Tg, 32>(x, st);
    case 64: return launch_bwd_t<Tin, Tg, 64>(x, st);
    default: return launch_bwd_t<Tin, Tg, 128>(x, st);
  }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& x, int d, int in_dt, int out_dt, hipStream_t st) {
  hipError_t e;
  if (in_dt == HLTA_BF16)
    e = out_dt == HLTA_BF16 ? launch_bwd_d<bf16, bf16>(x, d, st) : launch_bwd_d<bf16, float>(x, d, st);
  else
    e = launch_bwd_d<float, float>(x, d, st);
  if (e != hipSuccess) return e;
  const long long ntok = (long long)x.attn.B * x.gdn.L;
  const dim3 pg(unsigned(x.attn.H), unsigned(x.dw_slices));
  if (out_dt == HLTA_BF16)
    hipLaunchKernelGGL((dmix_partial<bf16, bf16>), pg, dim3(kThreads), 0, st, static_cast<const bf16*>(x.d_mix),
                       static_cast<const bf16*>(x.o_swa), static_cast<const bf16*>(x.o_dswa),
                       static_cast<const bf16*>(x.o_gdn), x.dw_part, ntok, x.attn.H, d);
  else
    hipLaunchKernelGGL((dmix_partial<float, float>), pg, dim3(kThreads), 0, st, static_cast<const float*>(x.d_mix),
                       static_cast<const float*>(x.o_swa), static_cast<const float*>(x.o_dswa),
                       static_cast<const float*>(x.o_gdn), x.dw_part, ntok, x.attn.H, d);
  hipLaunchKernelGGL(dmix_final, dim3(unsigned((3 * x.attn.H + 63) / 64)), dim3(64), 0, st, x.dw_part, x.dmix_w,
                     x.attn.H, x.dw_slices);
  return hipGetLastError();
}

}  // namespace hlta
