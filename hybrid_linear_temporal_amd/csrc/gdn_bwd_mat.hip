// Backward of the gated delta rule, chunk by chunk in matrix (UT / WY) form
// (Kairos related-work page, row A: the gated delta rule; long-context page,
// sections 02 and 06: chunkwise-parallel and recurrent forms of such a state
// are equivalent algorithms, and section 06 on chunking with the WY / UT
// transform). fp32 values, products on bf16 MFMA with split (hi + lo) factors
// (close to fp32 accuracy), any supported d, chunks of C <= 64 tokens.
//
// Inside one chunk (rows t < n; the chunk is zero-padded to 64 rows, which
// leaves every product below unchanged), with k^, q^ the normalised keys and
// queries, g_i = sum_{j<=i} log a_j, gamma_i = exp(g_i), gamma_C = gamma at the
// chunk's last row, Gam_ij = exp(g_i - g_j) (j <= i), the forward is
//   A = strict_lower(diag(b) (Gam . K K^T)),  T = (I + A)^-1,
//   W = T diag(b gamma) K,  U' = T diag(b) V,  U = U' - W S^T,
//   P = lower(Gam . Q K^T),  O = diag(gamma) Q S^T + P U,
//   S_end = S M + N,  M = gamma_C I - W^T De K,  N = U'^T De K,  De = diag(gamma_C / gamma).
// The adjoint reaching the chunk's start is dS = G M^T + X with
// X = dO^T (diag(gamma) Q - P W), G the adjoint at its end. Given S (start
// state) and G, the gradients of the chunk's tokens are
//   dU = P^T dO + De K G^T,  dP = lower(dO U^T),
//   dq^ = diag(gamma) dO S + (dP . Gam) K,  dW = -dU S,
//   dv = diag(b) T^T dU,  dT = dW (diag(b gamma) K)^T + dU (diag(b) V)^T,
//   dA = strict_lower(-T^T dT T^T),  dKK = dA . (b_i Gam_ij),
//   dk^ = (dP . Gam)^T Q + De U G + diag(b gamma) T^T dW + dKK K + dKK^T K,
//   db_i = gamma_i (T^T dW)_i . k_i + (T^T dU)_i . v_i + sum_j dA_ij (Gam . KK)_ij,
// and, with E = dA . A + dP . P, the log-gate prefix sums get
//   dg_i = sum_j E_ij - sum_j E_ji + b_i gamma_i (T^T dW)_i . k_i
//          + gamma_i q_i . (dO S)_i - t_i,   t_i = U_i . (De K G^T)_i,
//   dg_last += gamma_C <G, S> + sum_i t_i;
// d(log a_t) = sum_{i >= t} dg_i and da_t = d(log a_t) / a_t. dq, dk then go
// through the L2 normalisation: dx = (dx^ - x^ (x^ . dx^)) / n(x).
//
// Two kernels replace a token-by-token walk: gdn_bwd_mat_prep (per chunk: M,
// M^T, N, X for the chains over chunks) and gdn_bwd_mat_grad (per chunk, after
// the chains: the token gradients). Each is a persistent grid, one workgroup
// per scratch slot of the workspace; the chunk's matrices live in that slot
// (global memory, resident in the caches) and every product goes through LDS
// to the matrix cores.
#include "hlta_device.h"
#include "hlta_internal.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kNT = 256;
constexpr int CM = 64;               // chunk rows
constexpr float kEps = 1e-6f;
constexpr float kLogFloor = -80.f;   // log a below this is clamped (a underflows)

// four consecutive values (8- or 16-byte aligned) as floats
__device__ __forceinline__ float4 ld4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4f(const bf16* p) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
  return make_float4(static_cast<float>(x[0]), static_cast<float>(x[1]), static_cast<float>(x[2]),
                     static_cast<float>(x[3]));
}

// C = alpha op(A) op(B) (+ C when acc): op(A) M x K, op(B) K x N, row-major
// with leading dimensions (multiples of 4, 16-byte aligned rows); TA: A is
// stored K x M, TB: B is stored N x K. Products on bf16 MFMA with each factor
// split into a high and a low bf16 part (x = hi + lo, about 16 significant
// bits): hi*hi + hi*lo + lo*hi in fp32 accumulation, so the result keeps
// close to fp32 accuracy. K goes through LDS in slices of 64, staged as the
// split parts in rows of 72 bf16 (k contiguous, 16-byte reads free of bank
// conflicts); wave w computes the 32 x 32 output tiles w, w + 4, .. with
// v_mfma_f32_32x32x16_bf16 (A: lane = row l%32, k 8(l/32) ..; B: lane =
// column l%32, same k; C: lane = column l%32, rows 8(r/4) + 4(l/32) + r%4).
// Ends with a barrier, so C is visible to the whole workgroup (C must not
// alias A or B).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kKS = 64;   // k per slice
constexpr int kRow = 72;  // bf16 per staged row (64 + pad)
constexpr int kLdsFloats = 4 * 128 * kRow / 2;   // hi and lo of A and B, up to 128 rows each

__device__ __forceinline__ void split_store(bf16* hi, bf16* lo, float x) {
  const bf16 h = static_cast<bf16>(x);
  *hi = h;
  *lo = static_cast<bf16>(x - static_cast<float>(h));
}
// four consecutive k of one row: one 8-byte store each for hi and lo
__device__ __forceinline__ void split_store4(bf16* hi, bf16* lo, const float4& x) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  const bf16x4_t h = {static_cast<bf16>(x.x), static_cast<bf16>(x.y), static_cast<bf16>(x.z), static_cast<bf16>(x.w)};
  const bf16x4_t l = {static_cast<bf16>(x.x - static_cast<float>(h[0])), static_cast<bf16>(x.y - static_cast<float>(h[1])),
                      static_cast<bf16>(x.z - static_cast<float>(h[2])), static_cast<bf16>(x.w - static_cast<float>(h[3]))};
  *reinterpret_cast<bf16x4_t*>(hi) = h;
  *reinterpret_cast<bf16x4_t*>(lo) = l;
}

template <int M, int N, int K, bool TA, bool TB>
__device__ __attribute__((noinline)) void mm(float* C, int ldc, const float* A, int lda, const float* B, int ldb,
                                             float alpha, bool acc, float* lds) {
  constexpr int KS = K < kKS ? K : kKS;   // k of one slice
  static_assert(M % 32 == 0 && N % 32 == 0 && K % KS == 0 && KS % 16 == 0 && M <= 128 && N <= 128, "aligned shapes");
  constexpr int NT = (M / 32) * (N / 32), TPW = (NT + 3) / 4;   // tiles, tiles per wave
  bf16* Ahi = reinterpret_cast<bf16*>(lds);
  bf16* Alo = Ahi + M * kRow;
  bf16* Bhi = Alo + M * kRow;
  bf16* Blo = Bhi + N * kRow;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  f32x16_t c[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[u][r] = 0.f;
  for (int k0 = 0; k0 < K; k0 += KS) {
    __syncthreads();
    for (int e = tid; e < M * KS / 4; e += kNT) {
      if (TA) {
        const int kk = e / (M / 4), i4 = e % (M / 4);
        const float4 x = *reinterpret_cast<const float4*>(A + size_t(k0 + kk) * lda + 4 * i4);
        split_store(Ahi + (4 * i4 + 0) * kRow + kk, Alo + (4 * i4 + 0) * kRow + kk, x.x);
        split_store(Ahi + (4 * i4 + 1) * kRow + kk, Alo + (4 * i4 + 1) * kRow + kk, x.y);
        split_store(Ahi + (4 * i4 + 2) * kRow + kk, Alo + (4 * i4 + 2) * kRow + kk, x.z);
        split_store(Ahi + (4 * i4 + 3) * kRow + kk, Alo + (4 * i4 + 3) * kRow + kk, x.w);
      } else {
        const int i = e / (KS / 4), k4 = e % (KS / 4);
        const float4 x = *reinterpret_cast<const float4*>(A + size_t(i) * lda + k0 + 4 * k4);
        split_store4(Ahi + i * kRow + 4 * k4, Alo + i * kRow + 4 * k4, x);
      }
    }
    for (int e = tid; e < N * KS / 4; e += kNT) {
      if (TB) {
        const int j = e / (KS / 4), k4 = e % (KS / 4);
        const float4 x = *reinterpret_cast<const float4*>(B + size_t(j) * ldb + k0 + 4 * k4);
        split_store4(Bhi + j * kRow + 4 * k4, Blo + j * kRow + 4 * k4, x);
      } else {
        const int kk = e / (N / 4), j4 = e % (N / 4);
        const float4 x = *reinterpret_cast<const float4*>(B + size_t(k0 + kk) * ldb + 4 * j4);
        split_store(Bhi + (4 * j4 + 0) * kRow + kk, Blo + (4 * j4 + 0) * kRow + kk, x.x);
        split_store(Bhi + (4 * j4 + 1) * kRow + kk, Blo + (4 * j4 + 1) * kRow + kk, x.y);
        split_store(Bhi + (4 * j4 + 2) * kRow + kk, Blo + (4 * j4 + 2) * kRow + kk, x.z);
        split_store(Bhi + (4 * j4 + 3) * kRow + kk, Blo + (4 * j4 + 3) * kRow + kk, x.w);
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wave + 4 * u;
      if (t < NT) {
        const int tm = t / (N / 32), tn = t % (N / 32);
#pragma unroll
        for (int ks = 0; ks < KS / 16; ++ks) {
          const int ko = 16 * ks + 8 * hl;
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(Ahi + (32 * tm + l32) * kRow + ko);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(Alo + (32 * tm + l32) * kRow + ko);
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(Bhi + (32 * tn + l32) * kRow + ko);
          const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(Blo + (32 * tn + l32) * kRow + ko);
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c[u], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + 4 * u;
    if (t < NT) {
      const int tm = t / (N / 32), tn = t % (N / 32);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tm + 8 * (r >> 2) + 4 * hl + (r & 3), col = 32 * tn + l32;
        float* cp = C + size_t(row) * ldc + col;
        *cp = alpha * c[u][r] + (acc ? *cp : 0.f);
      }
    }
  }
  __syncthreads();
}

// out[t] = sum_j X[t][j] Y[t][j], t < CM (a wave per row, lanes over columns)
template <int D>
__device__ void rowdot(float* out, const float* X, const float* Y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int t = wave; t < CM; t += kNT / 64) {
    float s = 0.f;
    for (int j = lane; j < D; j += 64) s += X[size_t(t) * D + j] * Y[size_t(t) * D + j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) out[t] = s;
  }
  __syncthreads();
}

// T = (I + diag(b) L)^-1 for strictly lower L [CM][CM] (global): L goes to
// LDS; four lanes per column j (lane q holds t_m for m = q mod 4) solve it by
// forward substitution, the partial dot products joined by two shuffles.
__device__ __attribute__((noinline)) void tri_inverse(float* Tm, const float* L, const float* b, float* lds) {
  for (int e = threadIdx.x; e < CM * CM / 4; e += kNT)
    reinterpret_cast<float4*>(lds)[e] = reinterpret_cast<const float4*>(L)[e];
  __syncthreads();
  const int j = threadIdx.x >> 2, q = threadIdx.x & 3;
  float t[CM / 4];
#pragma unroll
  for (int r = 0; r < CM / 4; ++r) t[r] = 0.f;
#pragma unroll
  for (int i = 0; i < CM; ++i) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < (i + 3) / 4; ++r) {
      const float l = 4 * r + q < i ? lds[i * CM + 4 * r + q] : 0.f;
      if (r & 1) s1 = fmaf(l, t[r], s1);
      else s0 = fmaf(l, t[r], s0);
    }
    float s = s0 + s1;
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const float ti = (i == j ? 1.f : 0.f) - b[i] * s;
    if ((i & 3) == q) t[i >> 2] = ti;
  }
#pragma unroll
  for (int r = 0; r < CM / 4; ++r) Tm[size_t(4 * r + q) * CM + j] = t[r];
  __syncthreads();
}

// Per-workgroup scratch (floats, in its slot of the workspace)
template <int D>
struct Slot {
  static constexpr size_t CD = size_t(CM) * D, CC = size_t(CM) * CM;
  static_assert(16 * CD + 7 * CC <= bwd_slot_floats(D), "the slot holds the chunk's matrices");
  static_assert(kLdsFloats >= CC, "the inverse's LDS fits the product staging");
  float* base;
  __device__ float* cd(int i) const { return base + i * CD; }            // [CM][D] matrices 0 ..
  __device__ float* cc(int i) const { return base + 16 * CD + i * CC; }  // [CM][CM] matrices 0 ..
};
// [CM][D] slots
enum { sK = 0, sQ, sV, sDO, sBK, sDK, sW, sUp, sU, sDU, sX1, sX2, sX3, sDKG, sBV };
// [CM][CM] slots
enum { sGK = 0, sT, sP, sDP, sDPG, sE1, sE2 };

// Chunk vectors in LDS
struct ChunkVec {
  float g[CM], gam[CM], De[CM], b[CM], a[CM], rk[CM], rq[CM];
  float v0[CM], v1[CM], v2[CM], v3[CM], v4[CM];
  float red[kNT / 64];
  float gC;
};

// Loads chunk c of head (b, h): K, Q (normalised), V, dO = w2 d_mix, gates,
// then forms diag(b gamma) K, De K, diag(b) V, strict_lower(Gam . K K^T), T,
// W, U' and P. Rows t >= n are zero (gates a = 1, b = 0).
template <typename Tin, typename Tg, int D>
__device__ void chunk_forward(const GdnParams& p, int C, const Tg* d_mix, float w2, int c, int b, int h,
                              const Slot<D>& s, ChunkVec& v, float* lds) {
  const size_t HD = size_t(p.H) * D;
  const long long t0 = (long long)c * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const size_t tok0 = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
  const size_t g0 = (size_t(b) * p.L + t0) * p.H + h;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* vv = static_cast<const Tin*>(p.v);
  float *K = s.cd(sK), *Q = s.cd(sQ), *V = s.cd(sV), *dO = s.cd(sDO);
  for (int e = threadIdx.x; e < CM * D / 4; e += kNT) {
    const int t = (4 * e) / D, j = (4 * e) % D;
    float4 xk = {0.f, 0.f, 0.f, 0.f}, xq = xk, xv = xk, xd = xk;
    if (t < n) {
      const size_t o = tok0 + size_t(t) * HD + j;
      xk = ld4f(k + o);
      xq = ld4f(q + o);
      xv = ld4f(vv + o);
      xd = ld4f(d_mix + o);
      xd = make_float4(w2 * xd.x, w2 * xd.y, w2 * xd.z, w2 * xd.w);
    }
    reinterpret_cast<float4*>(K)[e] = xk;
    reinterpret_cast<float4*>(Q)[e] = xq;
    reinterpret_cast<float4*>(V)[e] = xv;
    reinterpret_cast<float4*>(dO)[e] = xd;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (wave == 0) {
    const int t = lane;
    const float at = t < n ? p.a[g0 + size_t(t) * p.H] : 1.f;
    const float bt = t < n ? p.b[g0 + size_t(t) * p.H] : 0.f;
    float la = at > 0.f ? fmaxf(logf(at), kLogFloor) : kLogFloor;
    if (t >= n) la = 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (lane >= off) la += y;
    }
    v.g[t] = la;
    v.gam[t] = expf(la);
    v.a[t] = at;
    v.b[t] = bt;
  }
  __syncthreads();   // K, Q written; gates
  {
    // norms: a wave per row, lanes over columns
    for (int t = wave; t < CM; t += kNT / 64) {
      float sk = 0.f, sq = 0.f;
      for (int j = lane; j < D; j += 64) {
        const float kx = K[size_t(t) * D + j], qx = Q[size_t(t) * D + j];
        sk += kx * kx;
        sq += qx * qx;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        sk += __shfl_xor(sk, off);
        sq += __shfl_xor(sq, off);
      }
      if (lane == 0) {
        v.rk[t] = p.l2norm ? 1.f / sqrtf(sk + kEps) : 1.f;
        v.rq[t] = p.l2norm ? 1.f / sqrtf(sq + kEps) : 1.f;
        v.De[t] = expf(v.g[CM - 1] - v.g[t]);
      }
    }
    if (threadIdx.x == 0) v.gC = v.gam[CM - 1];
  }
  __syncthreads();
  float *BK = s.cd(sBK), *DK = s.cd(sDK), *BV = s.cd(sBV);
  for (int e = threadIdx.x; e < CM * D; e += kNT) {
    const int t = e / D;
    const float kx = K[e] * v.rk[t];
    K[e] = kx;
    Q[e] *= v.rq[t];
    BK[e] = v.b[t] * v.gam[t] * kx;
    DK[e] = v.De[t] * kx;
    BV[e] = v.b[t] * V[e];
  }
  __syncthreads();
  // GK = strict_lower(Gam . K K^T), T = (I + diag(b) GK)^-1
  float *GK = s.cc(sGK), *Tm = s.cc(sT), *P = s.cc(sP);
  mm<CM, CM, D, false, true>(GK, CM, K, D, K, D, 1.f, false, lds);
  for (int e = threadIdx.x; e < CM * CM; e += kNT) {
    const int i = e / CM, j = e % CM;
    GK[e] = j < i ? expf(v.g[i] - v.g[j]) * GK[e] : 0.f;
  }
  __syncthreads();
  tri_inverse(Tm, GK, v.b, lds);
  mm<CM, D, CM, false, false>(s.cd(sW), D, Tm, CM, BK, D, 1.f, false, lds);
  mm<CM, D, CM, false, false>(s.cd(sUp), D, Tm, CM, BV, D, 1.f, false, lds);
  // P = lower(Gam . Q K^T)
  mm<CM, CM, D, false, true>(P, CM, Q, D, K, D, 1.f, false, lds);
  for (int e = threadIdx.x; e < CM * CM; e += kNT) {
    const int i = e / CM, j = e % CM;
    P[e] = j <= i ? expf(v.g[i] - v.g[j]) * P[e] : 0.f;
  }
  __syncthreads();
}

// Per chunk: M (Am), M^T (AmT), N (Um) and the chunk's own adjoint X (Xm).
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kNT)
gdn_bwd_mat_prep(GdnParams p, int C, const Tg* d_mix, const float* mix_w, float* slots, size_t slot_floats,
                 float* Am, float* AmT, float* Um, float* Xm) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];   // product staging or the inverse
  __shared__ ChunkVec v;
  const Slot<D> s{slots + size_t(blockIdx.x) * slot_floats};
  const long long jobs = (long long)p.B * p.H * p.n_chunks;
  const size_t mat = size_t(D) * D;
  for (long long job = blockIdx.x; job < jobs; job += gridDim.x) {
    const int c = int(job % p.n_chunks), bh = int(job / p.n_chunks), b = bh / p.H, h = bh % p.H;
    chunk_forward<Tin, Tg, D>(p, C, d_mix, mix_w[3 * h + 2], c, b, h, s, v, lds);
    float *W = s.cd(sW), *Up = s.cd(sUp), *DK = s.cd(sDK), *Q = s.cd(sQ), *dO = s.cd(sDO), *Y = s.cd(sX1);
    float* am = Am + size_t(job) * mat;
    float* amt = AmT + size_t(job) * mat;
    mm<D, D, CM, true, false>(am, D, W, D, DK, D, -1.f, false, lds);    // -W^T De K
    mm<D, D, CM, true, false>(amt, D, DK, D, W, D, -1.f, false, lds);   // -K^T De W
    mm<D, D, CM, true, false>(Um + size_t(job) * mat, D, Up, D, DK, D, 1.f, false, lds);
    for (int i = threadIdx.x; i < D; i += kNT) {
      am[size_t(i) * D + i] += v.gC;
      amt[size_t(i) * D + i] += v.gC;
    }
    // X = dO^T (diag(gamma) Q - P W)
    mm<CM, D, CM, false, false>(Y, D, s.cc(sP), CM, W, D, -1.f, false, lds);
    for (int e = threadIdx.x; e < CM * D; e += kNT) Y[e] += v.gam[e / D] * Q[e];
    __syncthreads();
    mm<D, D, CM, true, false>(Xm + size_t(job) * mat, D, dO, D, Y, D, 1.f, false, lds);
  }
}

// Per chunk, given its start state S (Sst) and the adjoint G reaching its end
// (Rin): dq, dk, dv (added to what the softmax branches wrote), da, db.
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kNT)
gdn_bwd_mat_grad(GdnParams p, int C, const Tg* d_mix, const float* mix_w, float* slots, size_t slot_floats,
                 const float* Sst, const float* Rin, float* dq, float* dk, float* dv, float* da, float* db) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
  __shared__ ChunkVec v;
  const Slot<D> s{slots + size_t(blockIdx.x) * slot_floats};
  const long long jobs = (long long)p.B * p.H * p.n_chunks;
  const size_t mat = size_t(D) * D;
  const size_t HD = size_t(p.H) * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (long long job = blockIdx.x; job < jobs; job += gridDim.x) {
    const int c = int(job % p.n_chunks), bh = int(job / p.n_chunks), b = bh / p.H, h = bh % p.H;
    const long long t0 = (long long)c * C;
    const int n = int(p.L - t0 < C ? p.L - t0 : C);
    const size_t tok0 = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
    const size_t g0 = (size_t(b) * p.L + t0) * p.H + h;
    chunk_forward<Tin, Tg, D>(p, C, d_mix, mix_w[3 * h + 2], c, b, h, s, v, lds);
    const float* S = Sst + size_t(job) * mat;
    const float* G = Rin + size_t(job) * mat;
    float *K = s.cd(sK), *Q = s.cd(sQ), *V = s.cd(sV), *dO = s.cd(sDO), *DK = s.cd(sDK), *BK = s.cd(sBK);
    float *W = s.cd(sW), *Up = s.cd(sUp), *U = s.cd(sU), *dU = s.cd(sDU), *DKG = s.cd(sDKG);
    float *X1 = s.cd(sX1), *X2 = s.cd(sX2), *X3 = s.cd(sX3), *BV = s.cd(sBV);
    float *GK = s.cc(sGK), *Tm = s.cc(sT), *P = s.cc(sP), *dP = s.cc(sDP), *dPG = s.cc(sDPG);
    float *E1 = s.cc(sE1), *E2 = s.cc(sE2);

    // U = U' - W S^T;  De K G^T;  t_i = U_i . (De K G^T)_i
    for (int e = threadIdx.x; e < CM * D; e += kNT) U[e] = Up[e];
    mm<CM, D, D, false, true>(U, D, W, D, S, D, -1.f, true, lds);
    mm<CM, D, D, false, true>(DKG, D, DK, D, G, D, 1.f, false, lds);
    rowdot<D>(v.v0, U, DKG);   // t_i
    // dU = P^T dO + De K G^T
    for (int e = threadIdx.x; e < CM * D; e += kNT) dU[e] = DKG[e];
    mm<CM, D, CM, true, false>(dU, D, P, CM, dO, D, 1.f, true, lds);
    // dP = lower(dO U^T), dPG = dP . Gam
    mm<CM, CM, D, false, true>(dP, CM, dO, D, U, D, 1.f, false, lds);
    for (int e = threadIdx.x; e < CM * CM; e += kNT) {
      const int i = e / CM, j = e % CM;
      const float x = j <= i ? dP[e] : 0.f;
      dP[e] = x;
      dPG[e] = j <= i ? x * expf(v.g[i] - v.g[j]) : 0.f;
    }
    __syncthreads();
    // dq^ = diag(gamma) dO S + dPG K (the row dots q_i . (dO S)_i first)
    mm<CM, D, D, false, false>(X1, D, dO, D, S, D, 1.f, false, lds);
    rowdot<D>(v.v1, X1, Q);   // q_i . (dO S)_i
    for (int e = threadIdx.x; e < CM * D; e += kNT) X1[e] *= v.gam[e / D];
    __syncthreads();
    mm<CM, D, CM, false, false>(X1, D, dPG, CM, K, D, 1.f, true, lds);
    // through the normalisation, into dq
    rowdot<D>(v.v2, X1, Q);   // q^ . dq^
    for (int e = threadIdx.x; e < n * D; e += kNT) {
      const int t = e / D, j = e % D;
      const float x = p.l2norm ? (X1[e] - Q[e] * v.v2[t]) * v.rq[t] : X1[e];
      dq[tok0 + size_t(t) * HD + j] += x;
    }
    __syncthreads();
    // dW = -dU S (X2), T^T dW (X3), dT = dW (diag(b gamma) K)^T (E1)
    mm<CM, D, D, false, false>(X2, D, dU, D, S, D, -1.f, false, lds);
    mm<CM, D, CM, true, false>(X3, D, Tm, CM, X2, D, 1.f, false, lds);
    mm<CM, CM, D, false, true>(E1, CM, X2, D, BK, D, 1.f, false, lds);
    // T^T dU (X2), dT += dU (diag(b) V)^T
    mm<CM, D, CM, true, false>(X2, D, Tm, CM, dU, D, 1.f, false, lds);
    mm<CM, CM, D, false, true>(E1, CM, dU, D, BV, D, 1.f, true, lds);
    // dv = diag(b) T^T dU; row dots for db
    for (int e = threadIdx.x; e < n * D; e += kNT) {
      const int t = e / D, j = e % D;
      dv[tok0 + size_t(t) * HD + j] += v.b[t] * X2[e];
    }
    rowdot<D>(v.v2, X2, V);   // (T^T dU)_i . v_i
    rowdot<D>(v.v3, X3, K);   // (T^T dW)_i . k_i
    // dA = strict_lower(-T^T dT T^T) (E1), via E2 = dT T^T
    mm<CM, CM, CM, false, true>(E2, CM, E1, CM, Tm, CM, 1.f, false, lds);
    mm<CM, CM, CM, true, false>(E1, CM, Tm, CM, E2, CM, -1.f, false, lds);
    // E2 = dKK = dA . (b_i Gam_ij); E (into dP) = dA . A + dP . P; db part sum_j dA GK
    for (int e = threadIdx.x; e < CM * CM; e += kNT) {
      const int i = e / CM, j = e % CM;
      const float dA = j < i ? E1[e] : 0.f;
      E1[e] = dA * GK[e];   // dA . (Gam . KK), row sums feed db
      E2[e] = j < i ? dA * v.b[i] * expf(v.g[i] - v.g[j]) : 0.f;
      dP[e] = dA * v.b[i] * GK[e] + dP[e] * P[e];
    }
    __syncthreads();
    // gates: row and column sums of E, the db row sums of dA . GK
    if (wave == 0) {
      float rs = 0.f, cs = 0.f, gs = 0.f;
      for (int j = 0; j < CM; ++j) {
        rs += dP[lane * CM + j];
        cs += dP[j * CM + lane];
        gs += E1[lane * CM + j];
      }
      v.v4[lane] = rs - cs;
      // db (before the gates' own terms overwrite the scratch)
      const float dbt = v.gam[lane] * v.v3[lane] + v.v2[lane] + gs;
      if (lane < n) db[g0 + size_t(lane) * p.H] = dbt;
    }
    // <G, S>
    {
      float x = 0.f;
      for (size_t e = threadIdx.x; e < mat; e += kNT) x += G[e] * S[e];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
      if (lane == 0) v.red[wave] = x;
    }
    __syncthreads();
    if (wave == 0) {
      const int i = lane;
      float tsum = v.v0[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tsum += __shfl_xor(tsum, off);
      float GS = 0.f;
      for (int w = 0; w < kNT / 64; ++w) GS += v.red[w];
      float dg = v.v4[i] + v.b[i] * v.gam[i] * v.v3[i] + v.gam[i] * v.v1[i] - v.v0[i];
      if (i == CM - 1) dg += v.gC * GS + tsum;
      // d(log a_t) = sum_{i >= t} dg_i
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(dg, off);
        if (i + off < 64) dg += y;
      }
      if (i < n) da[g0 + size_t(i) * p.H] = v.a[i] > 0.f ? dg / v.a[i] : 0.f;
    }
    // dk^ = De U G + diag(b gamma) T^T dW + dPG^T Q + dKK K + dKK^T K
    mm<CM, D, D, false, false>(X1, D, U, D, G, D, 1.f, false, lds);
    for (int e = threadIdx.x; e < CM * D; e += kNT) {
      const int t = e / D;
      X1[e] = v.De[t] * X1[e] + v.b[t] * v.gam[t] * X3[e];
    }
    __syncthreads();
    mm<CM, D, CM, true, false>(X1, D, dPG, CM, Q, D, 1.f, true, lds);
    mm<CM, D, CM, false, false>(X1, D, E2, CM, K, D, 1.f, true, lds);
    mm<CM, D, CM, true, false>(X1, D, E2, CM, K, D, 1.f, true, lds);
    rowdot<D>(v.v2, X1, K);   // k^ . dk^
    for (int e = threadIdx.x; e < n * D; e += kNT) {
      const int t = e / D, j = e % D;
      const float x = p.l2norm ? (X1[e] - K[e] * v.v2[t]) * v.rk[t] : X1[e];
      dk[tok0 + size_t(t) * HD + j] += x;
    }
    __syncthreads();
  }
}

template <typename Tin, typename Tg, int D>
hipError_t launch_t(const BwdArgs& x, int phase, hipStream_t st) {
  const Tg* g = static_cast<const Tg*>(x.d_mix);
  const dim3 grid(unsigned(x.n_slots));
  if (phase == 0)
    hipLaunchKernelGGL((gdn_bwd_mat_prep<Tin, Tg, D>), grid, dim3(kNT), 0, st, x.gdn, x.C, g, x.mix_w, x.slots,
                       x.slot_floats, x.Am, x.AmT, x.Um, x.Xm);
  else
    hipLaunchKernelGGL((gdn_bwd_mat_grad<Tin, Tg, D>), grid, dim3(kNT), 0, st, x.gdn, x.C, g, x.mix_w, x.slots,
                       x.slot_floats, x.Sst, x.Rin, x.dq, x.dk, x.dv, x.da, x.db);
  return hipGetLastError();
}

template <typename Tin, typename Tg>
hipError_t launch_d(const BwdArgs& x, int d, int phase, hipStream_t st) {
  switch (d) {
    case 32: return launch_t<Tin, Tg, 32>(x, phase, st);
    case 64: return launch_t<Tin, Tg, 64>(x, phase, st);
    default: return launch_t<Tin, Tg, 128>(x, phase, st);
  }
}

}  // namespace

hipError_t launch_gdn_bwd_mat(const BwdArgs& x, int d, int in_dt, int out_dt, int phase, hipStream_t st) {
  if (in_dt == HLTA_BF16)
    return out_dt == HLTA_BF16 ? launch_d<bf16, bf16>(x, d, phase, st) : launch_d<bf16, float>(x, d, phase, st);
  return launch_d<float, float>(x, d, phase, st);
}

}  // namespace hlta
