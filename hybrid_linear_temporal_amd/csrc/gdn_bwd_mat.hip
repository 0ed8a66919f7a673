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
// N, X for the chains over chunks) and gdn_bwd_mat_grad (per chunk, after
// the chains: the token gradients). Each is a persistent grid walking the
// chunks; every chunk has a slot of the workspace (global memory) for its
// matrices: the prep kernel forms the chunk's forward ones there (normalised
// K and Q, V, dO, the gated copies, W, U', GK, P, T and the inverse norms),
// the gradient kernel reads them back and adds its own. Every product goes
// through LDS to the matrix cores.
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

// C = alpha op(A) op(B) (+ Z when Z is given; Z may be C itself): op(A)
// M x K, op(B) K x N, Z M x N, row-major
// with leading dimensions (multiples of 4, 16-byte aligned rows); TA: A is
// stored K x M, TB: B is stored N x K. Products on bf16 MFMA with each factor
// split into a high and a low bf16 part (x = hi + lo, about 16 significant
// bits): hi*hi + hi*lo + lo*hi in fp32 accumulation, so the result keeps
// close to fp32 accuracy. K goes through LDS in slices of up to 64; a slice's
// fp32 operands are loaded in batches of eight 16-byte loads per thread (all
// in flight together), split, and staged in the layout they are stored in,
// so every staging store writes four consecutive values:
//  * an operand stored with k contiguous (A: M x K, B: N x K) as rows of 72
//    bf16 (one row per output row or column; 16-byte reads of 8 consecutive
//    k, free of bank conflicts);
//  * an operand stored with k as its rows (A: K x M, B: K x N) as k-major rows
//    of M (N) bf16, read with ds_read_b64_tr_b16, which gives each lane four
//    consecutive k of its own column; the 8-byte chunks of a row are
//    XOR-permuted by the row's index mod 4 so the four rows of one read hit
//    distinct banks.
// Wave w computes the 32 x 32 output tiles w, w + 4, .. with
// v_mfma_f32_32x32x16_bf16 (A: lane = row l%32, k 8(l/32) ..; B: lane =
// column l%32, same k; C: lane = column l%32, rows 8(r/4) + 4(l/32) + r%4).
// Ends with a barrier, so C is visible to the whole workgroup (C must not
// alias A or B).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
constexpr int kKS = 64;   // k per slice
constexpr int kRow = 72;  // bf16 per staged row (64 + pad)
constexpr int kLdsFloats = 4 * 128 * kRow / 2;   // hi and lo of A and B, up to 128 rows each

// four consecutive values: one 8-byte store each for hi and lo
__device__ __forceinline__ void split_store4(bf16* hi, bf16* lo, const float4& x) {
  const bf16x4_t h = {static_cast<bf16>(x.x), static_cast<bf16>(x.y), static_cast<bf16>(x.z), static_cast<bf16>(x.w)};
  const bf16x4_t l = {static_cast<bf16>(x.x - static_cast<float>(h[0])), static_cast<bf16>(x.y - static_cast<float>(h[1])),
                      static_cast<bf16>(x.z - static_cast<float>(h[2])), static_cast<bf16>(x.w - static_cast<float>(h[3]))};
  *reinterpret_cast<bf16x4_t*>(hi) = h;
  *reinterpret_cast<bf16x4_t*>(lo) = l;
}

// k-major staging of an operand with W columns: element (k, m) of the slice
// sits in row k at 8-byte chunk (m / 4) ^ kmaj_sw(k), value m % 4.
template <int W>
__device__ __forceinline__ int kmaj_sw(int k) {
  return W == 128 ? 8 * (k & 3) : (W == 64 ? 8 * ((k & 3) >> 1) : 0);
}
template <int W>
__device__ __forceinline__ int kmaj_off(int k, int m) {   // bf16 offset of chunk start
  return k * W + 4 * ((m >> 2) ^ kmaj_sw<W>(k));
}
// Operand of one MFMA from k-major staging: lane l gets column c0 + l%32 and
// k = k0 + 8 (l / 32) .. + 7 (two transposed 8-byte reads of four k each).
template <int W>
__device__ __forceinline__ bf16x8_t ld_kmaj(const bf16* st, int k0, int c0, int lane) {
  const int j = lane & 15, e = j >> 2, q = j & 3;
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * q;   // first of this lane's four addressed columns
  const int kb = k0 + 8 * (lane >> 5);
  const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(st + kmaj_off<W>(kb + e, col)));
  const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(st + kmaj_off<W>(kb + 4 + e, col)));
  return bf16x8_t{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <int M, int N>
constexpr int mm_tpw() { return ((M / 32) * (N / 32) + 3) / 4; }   // 32 x 32 output tiles per wave

__device__ __forceinline__ float4 operator*(float s, const float4& x) { return make_float4(s * x.x, s * x.y, s * x.z, s * x.w); }

// Accumulates sa op(A) op(B) into the wave's output tiles c (sa = +-1, applied
// to A's values as they are staged, so exactly).
template <int M, int N, int K, bool TA, bool TB>
__device__ __forceinline__ void mm_term(f32x16_t (&c)[((M / 32) * (N / 32) + 3) / 4], const float* A, int lda, const float* B,
                                        int ldb, float sa, float* lds) {
  constexpr int KS = K < kKS ? K : kKS;   // k of one slice
  static_assert(M % 32 == 0 && N % 32 == 0 && K % KS == 0 && KS % 16 == 0 && M <= 128 && N <= 128, "aligned shapes");
  constexpr int NT = (M / 32) * (N / 32), TPW = mm_tpw<M, N>();
  constexpr int NA = M * KS / 4 / kNT, NB = N * KS / 4 / kNT;   // float4 of A and B per thread per slice
  static_assert(NA * kNT * 4 == M * KS && NB * kNT * 4 == N * KS, "slices split evenly over the threads");
  constexpr int SA = TA ? KS * M : M * kRow, SB = TB ? N * kRow : KS * N;   // bf16 per staged part
  static_assert(2 * (SA + SB) <= 2 * kLdsFloats, "staging fits");
  bf16* Ahi = reinterpret_cast<bf16*>(lds);
  bf16* Alo = Ahi + SA;
  bf16* Bhi = Alo + SA;
  bf16* Blo = Bhi + SB;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  // staging in rounds of at most 8 float4 per thread (A's first, then B's),
  // each round's loads in flight together
  constexpr int kBatch = 8;
#pragma unroll 1
  for (int k0 = 0; k0 < K; k0 += KS) {
    __syncthreads();   // the previous slice's products are done with the staging area
#pragma unroll
    for (int u0 = 0; u0 < NA + NB; u0 += kBatch) {
      float4 x[kBatch];
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int u = u0 + v;
        if (u < NA) {
          const int e = tid + u * kNT;
          if (TA) {
            const int kk = e / (M / 4), i4 = e % (M / 4);
            x[v] = *reinterpret_cast<const float4*>(A + size_t(k0 + kk) * lda + 4 * i4);
          } else {
            const int i = e / (KS / 4), k4 = e % (KS / 4);
            x[v] = *reinterpret_cast<const float4*>(A + size_t(i) * lda + k0 + 4 * k4);
          }
        } else if (u < NA + NB) {
          const int e = tid + (u - NA) * kNT;
          if (TB) {
            const int j = e / (KS / 4), k4 = e % (KS / 4);
            x[v] = *reinterpret_cast<const float4*>(B + size_t(j) * ldb + k0 + 4 * k4);
          } else {
            const int kk = e / (N / 4), j4 = e % (N / 4);
            x[v] = *reinterpret_cast<const float4*>(B + size_t(k0 + kk) * ldb + 4 * j4);
          }
        }
      }
#pragma unroll
      for (int v = 0; v < kBatch; ++v) {
        const int u = u0 + v;
        if (u < NA) {
          const int e = tid + u * kNT;
          if (TA) {
            const int kk = e / (M / 4), i4 = e % (M / 4);
            const int o = kmaj_off<M>(kk, 4 * i4);
            split_store4(Ahi + o, Alo + o, sa * x[v]);
          } else {
            const int i = e / (KS / 4), k4 = e % (KS / 4);
            split_store4(Ahi + i * kRow + 4 * k4, Alo + i * kRow + 4 * k4, sa * x[v]);
          }
        } else if (u < NA + NB) {
          const int e = tid + (u - NA) * kNT;
          if (TB) {
            const int j = e / (KS / 4), k4 = e % (KS / 4);
            split_store4(Bhi + j * kRow + 4 * k4, Blo + j * kRow + 4 * k4, x[v]);
          } else {
            const int kk = e / (N / 4), j4 = e % (N / 4);
            const int o = kmaj_off<N>(kk, 4 * j4);
            split_store4(Bhi + o, Blo + o, x[v]);
          }
        }
      }
    }
    __syncthreads();
    // k steps outermost and only partly unrolled, so the operand reads of a
    // step are not all hoisted at once (the register file holds two workgroups)
#pragma unroll 2
    for (int ks = 0; ks < KS / 16; ++ks) {
      const int ko = 16 * ks + 8 * hl;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int t = wave + 4 * u;
        if (t < NT) {
          const int tm = t / (N / 32), tn = t % (N / 32);
          bf16x8_t ah, al, bh, bl;
          if (TA) {
            ah = ld_kmaj<M>(Ahi, 16 * ks, 32 * tm, lane);
            al = ld_kmaj<M>(Alo, 16 * ks, 32 * tm, lane);
          } else {
            ah = *reinterpret_cast<const bf16x8_t*>(Ahi + (32 * tm + l32) * kRow + ko);
            al = *reinterpret_cast<const bf16x8_t*>(Alo + (32 * tm + l32) * kRow + ko);
          }
          if (TB) {
            bh = *reinterpret_cast<const bf16x8_t*>(Bhi + (32 * tn + l32) * kRow + ko);
            bl = *reinterpret_cast<const bf16x8_t*>(Blo + (32 * tn + l32) * kRow + ko);
          } else {
            bh = ld_kmaj<N>(Bhi, 16 * ks, 32 * tn, lane);
            bl = ld_kmaj<N>(Blo, 16 * ks, 32 * tn, lane);
          }
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, c[u], 0, 0, 0);
          c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, c[u], 0, 0, 0);
        }
      }
    }
  }
}

// C = alpha c + Z (Z may be C itself or null), then a barrier
template <int M, int N>
__device__ __forceinline__ void mm_store(const f32x16_t (&c)[((M / 32) * (N / 32) + 3) / 4], float* C, int ldc, float alpha,
                                         const float* Z) {
  constexpr int NT = (M / 32) * (N / 32), TPW = mm_tpw<M, N>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int t = wave + 4 * u;
    if (t < NT) {
      const int tm = t / (N / 32), tn = t % (N / 32);
      const size_t c0 = size_t(32 * tm + 4 * hl) * ldc + 32 * tn + l32;
      auto at = [&](int r) { return c0 + size_t(8 * (r >> 2) + (r & 3)) * ldc; };
      float z[16];   // all 16 addends in flight before the first store
#pragma unroll
      for (int r = 0; r < 16; ++r) z[r] = Z ? Z[at(r)] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) C[at(r)] = alpha * c[u][r] + z[r];
    }
  }
  __syncthreads();
}


template <int M, int N, int K, bool TA, bool TB>
__device__ __attribute__((noinline)) void mm(float* C, int ldc, const float* A, int lda, const float* B, int ldb,
                                             float alpha, const float* Z, float* lds) {
  f32x16_t c[mm_tpw<M, N>()];
#pragma unroll
  for (int u = 0; u < mm_tpw<M, N>(); ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[u][r] = 0.f;
  mm_term<M, N, K, TA, TB>(c, A, lda, B, ldb, 1.f, lds);
  mm_store<M, N>(c, C, ldc, alpha, Z);
}

// [GK; P] = [K; Q] K^T with the causal gate factors applied as they are
// stored: GK_ij = exp(g_i - g_j) (K K^T)_ij for j < i, P_ij = exp(g_i - g_j)
// (Q K^T)_ij for j <= i, 0 elsewhere; GK also goes to LDS (at lds, CM x CM)
// for the triangular solve that follows. K and Q are adjacent [CM][D] arrays.
template <int D>
__device__ __attribute__((noinline)) void gk_p(float* GKP, const float* KQ, const float* g, float* lds) {
  constexpr int M = 2 * CM, N = CM;
  f32x16_t c[mm_tpw<M, N>()];
#pragma unroll
  for (int u = 0; u < mm_tpw<M, N>(); ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[u][r] = 0.f;
  mm_term<M, N, D, false, true>(c, KQ, D, KQ, D, 1.f, lds);
  __syncthreads();   // the staging area becomes the solve's copy of GK
  constexpr int NT = (M / 32) * (N / 32);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int u = 0; u < mm_tpw<M, N>(); ++u) {
    const int t = wave + 4 * u;
    if (t < NT) {
      const int tm = t / (N / 32), tn = t % (N / 32);
      const int j = 32 * tn + l32;
      const float gj = g[j];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tm + 8 * (r >> 2) + 4 * hl + (r & 3), i = row % CM;
        const bool keep = row < CM ? j < i : j <= i;
        const float x = keep ? expf(g[i] - gj) * c[u][r] : 0.f;
        GKP[size_t(row) * N + j] = x;
        if (row < CM) lds[row * CM + j] = x;
      }
    }
  }
  __syncthreads();
}

// C = sa1 op(A1) op(B1) + sa2 op(A2) op(B2) (+ Z): two products summed in the
// accumulators (one pass over C instead of two); sa1, sa2 = +-1.
template <int M, int N, int K1, bool TA1, bool TB1, int K2, bool TA2, bool TB2>
__device__ __attribute__((noinline)) void mm2(float* C, int ldc, const float* A1, int lda1, const float* B1, int ldb1,
                                              float sa1, const float* A2, int lda2, const float* B2, int ldb2,
                                              float sa2, const float* Z, float* lds) {
  f32x16_t c[mm_tpw<M, N>()];
#pragma unroll
  for (int u = 0; u < mm_tpw<M, N>(); ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[u][r] = 0.f;
  mm_term<M, N, K1, TA1, TB1>(c, A1, lda1, B1, ldb1, sa1, lds);
  mm_term<M, N, K2, TA2, TB2>(c, A2, lda2, B2, ldb2, sa2, lds);
  mm_store<M, N>(c, C, ldc, 1.f, Z);
}

// Elementwise passes over the chunk's arrays as 16-byte vectors: ld(e)
// gathers what position e needs (returns a small struct), st(e, x) writes the
// results; each thread takes positions tid, tid + 256, .. and issues the
// loads of kBatch positions before the first store, so their latencies
// overlap (the arrays live in the workspace, mostly beyond the caches).
template <int N4, int kBatch, typename LD, typename ST>
__device__ __forceinline__ void ew(LD ld, ST st) {
  static_assert(N4 % kNT == 0, "whole passes");
  constexpr int PER = N4 / kNT;
  using X = decltype(ld(0));
  // an opaque copy of the thread index: addresses are formed here, not shared
  // with (and kept live from) other passes
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int u0 = 0; u0 < PER; u0 += kBatch) {
    X x[kBatch];
#pragma unroll
    for (int v = 0; v < kBatch; ++v)
      if (u0 + v < PER) x[v] = ld(tid + (u0 + v) * kNT);
#pragma unroll
    for (int v = 0; v < kBatch; ++v)
      if (u0 + v < PER) st(tid + (u0 + v) * kNT, x[v]);
    __builtin_amdgcn_sched_barrier(0);   // the next batch's loads stay behind these stores
  }
}
struct F4x2 { float4 a, b; };
struct F4x3 { float4 a, b, c; };
struct F4x4 { float4 a, b, c, d; };
__device__ __forceinline__ float4 operator+(const float4& x, const float4& y) {
  return make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
}
__device__ __forceinline__ float4 operator-(const float4& x, const float4& y) {
  return make_float4(x.x - y.x, x.y - y.y, x.z - y.z, x.w - y.w);
}
__device__ __forceinline__ float dot4(const float4& x, const float4& y) {
  return x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
}
__device__ __forceinline__ float4* f4(float* p) { return reinterpret_cast<float4*>(p); }
__device__ __forceinline__ const float4* f4(const float* p) { return reinterpret_cast<const float4*>(p); }

// out[t] = sum_j X[t][j] Y[t][j] for the W-wide rows t < CM: row t's W/4
// vectors go to W/4 consecutive lanes, all of a thread's loads in flight
// together, the partial sums joined by shuffles.
template <int W>
__device__ void rowdot(float* out, const float* X, const float* Y) {
  constexpr int LPR = W / 4, RPP = kNT / LPR, PASSES = CM / RPP, HALF = PASSES > 4 ? PASSES / 2 : PASSES;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));   // addresses formed here (see ew)
  const int c4 = tid % LPR, r0 = tid / LPR;
#pragma unroll
  for (int q0 = 0; q0 < PASSES; q0 += HALF) {
    float4 x[HALF], y[HALF];
#pragma unroll
    for (int q = 0; q < HALF; ++q) {
      x[q] = f4(X)[(r0 + (q0 + q) * RPP) * LPR + c4];
      y[q] = f4(Y)[(r0 + (q0 + q) * RPP) * LPR + c4];
    }
#pragma unroll
    for (int q = 0; q < HALF; ++q) {
      float d = dot4(x[q], y[q]);
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) d += __shfl_xor(d, off);
      if (c4 == 0) out[r0 + (q0 + q) * RPP] = d;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
}

// T = (I + diag(b) L)^-1 for strictly lower L [CM][CM] (in LDS), by forward
// substitution down the rows: one wave, lane j holding column j of T in
// registers; row i's L entries are read as broadcast 16-byte vectors (the
// zeros on and above the diagonal included, against t's not-yet-formed zeros)
// and summed in four chains, the newest t entering last.
__device__ __attribute__((noinline)) void tri_inverse(float* Tm, const float* b, const float* lds) {
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    float t[CM];
#pragma unroll
    for (int i = 0; i < CM; ++i) t[i] = 0.f;
#pragma unroll
    for (int i = 0; i < CM; ++i) {
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int r = 0; r < (i + 3) / 4; ++r) {
        const float4 l = f4(lds + i * CM)[r];
        s0 = fmaf(l.x, t[4 * r], s0);
        s1 = fmaf(l.y, t[4 * r + 1], s1);
        s2 = fmaf(l.z, t[4 * r + 2], s2);
        s3 = fmaf(l.w, t[4 * r + 3], s3);
      }
      t[i] = (i == j ? 1.f : 0.f) - b[i] * ((s0 + s1) + (s2 + s3));
    }
#pragma unroll
    for (int i = 0; i < CM; ++i) Tm[size_t(i) * CM + j] = t[i];
  }
  __syncthreads();
}

// A chunk's matrices (floats, in its slot of the workspace)
template <int D>
struct Slot {
  static constexpr size_t CD = size_t(CM) * D, CC = size_t(CM) * CM;
  static_assert(16 * CD + 7 * CC <= bwd_slot_floats(D) && 2 * CM <= CD, "the slot holds the chunk's matrices");
  static_assert(kLdsFloats >= CC, "the inverse's LDS fits the product staging");
  float* base;
  __device__ float* cd(int i) const { return base + i * CD; }            // [CM][D] matrices 0 ..
  __device__ float* cc(int i) const { return base + 16 * CD + i * CC; }  // [CM][CM] matrices 0 ..
};
// [CM][D] slots
// (K, Q adjacent: one product forms K K^T and Q K^T; dO, dU adjacent and X1, X2
// adjacent: one product forms dO S and dU S)
// (sRN: the inverse norms of k and q, 2 x CM floats)
enum { sK = 0, sQ, sV, sDO, sDU, sBK, sDK, sW, sUp, sU, sX1, sX2, sX3, sDKG, sBV, sRN };
// [CM][CM] slots
enum { sGK = 0, sP, sT, sDP, sDPG, sE1, sE2 };   // GK, P adjacent

// Chunk vectors in LDS
struct ChunkVec {
  float g[CM], gam[CM], De[CM], b[CM], a[CM], rk[CM], rq[CM];
  float v0[CM], v1[CM], v2[CM], v3[CM], v4[CM], gs[CM];
  float cpart[kNT / 64][CM];   // per-wave partial column sums
  float red[kNT / 64];
  float gC;
};

// The chunk's gate vectors (wave 0): prefix sums g of log a, gamma, a, b,
// De = gamma_C / gamma and gamma_C; rows t >= n get a = 1, b = 0.
__device__ void chunk_gates(const GdnParams& p, int C, int c, int b, int h, ChunkVec& v) {
  if (threadIdx.x >= 64) return;
  const long long t0 = (long long)c * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const size_t g0 = (size_t(b) * p.L + t0) * p.H + h;
  const int t = threadIdx.x;
  const float at = t < n ? p.a[g0 + size_t(t) * p.H] : 1.f;
  const float bt = t < n ? p.b[g0 + size_t(t) * p.H] : 0.f;
  float la = at > 0.f ? fmaxf(logf(at), kLogFloor) : kLogFloor;
  if (t >= n) la = 0.f;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(la, off);
    if (t >= off) la += y;
  }
  const float gl = __shfl(la, CM - 1);
  v.g[t] = la;
  v.gam[t] = expf(la);
  v.a[t] = at;
  v.b[t] = bt;
  v.De[t] = expf(gl - la);
  if (t == 0) v.gC = expf(gl);
}

// Loads chunk c of head (b, h) into its slot: K, Q (normalised), V, dO = w2 d_mix, gates,
// then forms diag(b gamma) K, De K, diag(b) V, strict_lower(Gam . K K^T), T,
// W, U', P and the inverse norms. Rows t >= n are zero (gates a = 1, b = 0).
template <typename Tin, typename Tg, int D>
__device__ void chunk_forward(const GdnParams& p, int C, const Tg* d_mix, float w2, int c, int b, int h,
                              const Slot<D>& s, ChunkVec& v, float* lds) {
  const size_t HD = size_t(p.H) * D;
  const long long t0 = (long long)c * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const size_t tok0 = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* vv = static_cast<const Tin*>(p.v);
  float *K = s.cd(sK), *Q = s.cd(sQ), *V = s.cd(sV), *dO = s.cd(sDO);
  float *BK = s.cd(sBK), *DK = s.cd(sDK), *BV = s.cd(sBV);
  chunk_gates(p, C, c, b, h, v);
  __syncthreads();
  // the inputs in one pass: K^, Q^ (each row's squared norm joined over the
  // D/4 consecutive lanes that hold the row), V, dO = w2 d_mix, and from them
  // diag(b gamma) K^, De K^, diag(b) V
  ew<CM * D / 4, 2>(
      [&](int e) {
        const int t = (4 * e) / D, j = (4 * e) % D;
        F4x4 x;
        x.a = x.b = x.c = x.d = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < n) {
          const size_t o = tok0 + size_t(t) * HD + j;
          x.a = ld4f(k + o);
          x.b = ld4f(q + o);
          x.c = ld4f(vv + o);
          x.d = ld4f(d_mix + o);
        }
        return x;
      },
      [&](int e, const F4x4& x) {
        const int t = (4 * e) / D;
        float sk = dot4(x.a, x.a), sq = dot4(x.b, x.b);
#pragma unroll
        for (int off = 1; off < D / 4; off <<= 1) {
          sk += __shfl_xor(sk, off);
          sq += __shfl_xor(sq, off);
        }
        const float rk = p.l2norm ? 1.f / sqrtf(sk + kEps) : 1.f;
        const float rq = p.l2norm ? 1.f / sqrtf(sq + kEps) : 1.f;
        if (e % (D / 4) == 0) {
          v.rk[t] = rk;
          v.rq[t] = rq;
        }
        const float4 kx = rk * x.a;
        f4(K)[e] = kx;
        f4(Q)[e] = rq * x.b;
        f4(V)[e] = x.c;
        f4(dO)[e] = w2 * x.d;
        f4(BK)[e] = (v.b[t] * v.gam[t]) * kx;
        f4(DK)[e] = v.De[t] * kx;
        f4(BV)[e] = v.b[t] * x.c;
      });
  __syncthreads();
  if (threadIdx.x < CM) {   // kept with the chunk's matrices for the gradient kernel
    float* rn = s.cd(sRN);
    rn[threadIdx.x] = v.rk[threadIdx.x];
    rn[CM + threadIdx.x] = v.rq[threadIdx.x];
  }
  // [GK; P] = [K; Q] K^T with masks and gate factors applied as stored
  // (GK = strict_lower(Gam . K K^T), P = lower(Gam . Q K^T)), then
  // T = (I + diag(b) GK)^-1 from GK's copy in LDS
  float *GK = s.cc(sGK), *Tm = s.cc(sT);
  static_assert(sQ == sK + 1 && sP == sGK + 1, "K, Q and GK, P adjacent");
  gk_p<D>(GK, K, v.g, lds);
  tri_inverse(Tm, v.b, lds);
  mm<CM, D, CM, false, false>(s.cd(sW), D, Tm, CM, BK, D, 1.f, nullptr, lds);
  mm<CM, D, CM, false, false>(s.cd(sUp), D, Tm, CM, BV, D, 1.f, nullptr, lds);
}

// Per chunk: M (Am), N (Um) and the chunk's own adjoint X (Xm).
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kNT, 2)
gdn_bwd_mat_prep(GdnParams p, int C, const Tg* d_mix, const float* mix_w, float* slots, size_t slot_floats,
                 float* Am, float* Um, float* Xm) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];   // product staging or the inverse
  __shared__ ChunkVec v;
  const long long jobs = (long long)p.B * p.H * p.n_chunks;
  const size_t mat = size_t(D) * D;
  for (long long job = blockIdx.x; job < jobs; job += gridDim.x) {
    const int c = int(job % p.n_chunks), bh = int(job / p.n_chunks), b = bh / p.H, h = bh % p.H;
    // the chunk's slot, its address opaque to the compiler, so it does not
    // hoist every per-thread address of the chunk's arrays out of the loop
    float* sb = slots + size_t(job) * slot_floats;
    asm volatile("" : "+s"(sb));
    const Slot<D> s{sb};
    chunk_forward<Tin, Tg, D>(p, C, d_mix, mix_w[3 * h + 2], c, b, h, s, v, lds);
    float *W = s.cd(sW), *Up = s.cd(sUp), *DK = s.cd(sDK), *Q = s.cd(sQ), *dO = s.cd(sDO), *Y = s.cd(sX1);
    float* am = Am + size_t(job) * mat;
    mm<D, D, CM, true, false>(am, D, W, D, DK, D, -1.f, nullptr, lds);    // -W^T De K
    mm<D, D, CM, true, false>(Um + size_t(job) * mat, D, Up, D, DK, D, 1.f, nullptr, lds);
    for (int i = threadIdx.x; i < D; i += kNT) am[size_t(i) * D + i] += v.gC;
    // X = dO^T (diag(gamma) Q - P W): Y = diag(gamma) Q first, then Y -= P W
    ew<CM * D / 4, 2>([&](int e) { return f4(Q)[e]; },
                      [&](int e, const float4& x) { f4(Y)[e] = v.gam[(4 * e) / D] * x; });
    __syncthreads();
    mm<CM, D, CM, false, false>(Y, D, s.cc(sP), CM, W, D, -1.f, Y, lds);
    mm<D, D, CM, true, false>(Xm + size_t(job) * mat, D, dO, D, Y, D, 1.f, nullptr, lds);
  }
}

// Per chunk, given its start state S (Sst) and the adjoint G reaching its end
// (Rin): dq, dk, dv (added to what the softmax branches wrote), da, db.
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kNT, 2)
gdn_bwd_mat_grad(GdnParams p, int C, const Tg* d_mix, const float* mix_w, float* slots, size_t slot_floats,
                 const float* Sst, const float* Rin, float* dq, float* dk, float* dv, float* da, float* db) {
  __shared__ __attribute__((aligned(16))) float lds[kLdsFloats];
  __shared__ ChunkVec v;
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
    float* sb = slots + size_t(job) * slot_floats;   // opaque (see gdn_bwd_mat_prep)
    asm volatile("" : "+s"(sb));
    const Slot<D> s{sb};
    // the chunk's forward matrices are in its slot (formed by the prep
    // kernel); only the gate vectors and inverse norms come to LDS again
    chunk_gates(p, C, c, b, h, v);
    if (threadIdx.x < CM) {
      const float* rn = s.cd(sRN);
      v.rk[threadIdx.x] = rn[threadIdx.x];
      v.rq[threadIdx.x] = rn[CM + threadIdx.x];
    }
    __syncthreads();
    const float* S = Sst + size_t(job) * mat;
    const float* G = Rin + size_t(job) * mat;
    float *K = s.cd(sK), *Q = s.cd(sQ), *V = s.cd(sV), *dO = s.cd(sDO), *DK = s.cd(sDK), *BK = s.cd(sBK);
    float *W = s.cd(sW), *Up = s.cd(sUp), *U = s.cd(sU), *dU = s.cd(sDU), *DKG = s.cd(sDKG);
    float *X1 = s.cd(sX1), *X2 = s.cd(sX2), *X3 = s.cd(sX3), *BV = s.cd(sBV);
    float *GK = s.cc(sGK), *Tm = s.cc(sT), *P = s.cc(sP), *dP = s.cc(sDP), *dPG = s.cc(sDPG);
    float *E1 = s.cc(sE1), *E2 = s.cc(sE2);
    // scatter-add of a [CM][D] array into a gradient (rows t < n), optionally
    // through the L2 normalisation's Jacobian (x^ the normalised rows, r the
    // inverse norms, pr[t] = x^_t . dx^_t)
    auto add_rows = [&](float* grad, const float* X, const float* Xh, const float* pr, const float* rn, bool norm) {
      ew<CM * D / 4, 2>(
          [&](int e) {
            const int t = (4 * e) / D, j = (4 * e) % D;
            F4x3 x;
            x.a = f4(X)[e];
            x.b = Xh ? f4(Xh)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
            x.c = t < n ? f4(grad)[(tok0 + size_t(t) * HD + j) / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
            return x;
          },
          [&](int e, const F4x3& x) {
            const int t = (4 * e) / D, j = (4 * e) % D;
            if (t >= n) return;
            const float4 d = norm ? rn[t] * (x.a - pr[t] * x.b) : (rn ? rn[t] * x.a : x.a);
            f4(grad)[(tok0 + size_t(t) * HD + j) / 4] = x.c + d;
          });
    };

    // U = U' - W S^T;  De K G^T;  t_i = U_i . (De K G^T)_i
    mm<CM, D, D, false, true>(U, D, W, D, S, D, -1.f, Up, lds);
    mm<CM, D, D, false, true>(DKG, D, DK, D, G, D, 1.f, nullptr, lds);
    rowdot<D>(v.v0, U, DKG);   // t_i
    // dU = P^T dO + De K G^T
    mm<CM, D, CM, true, false>(dU, D, P, CM, dO, D, 1.f, DKG, lds);
    // dP = lower(dO U^T), dPG = dP . Gam
    mm<CM, CM, D, false, true>(dP, CM, dO, D, U, D, 1.f, nullptr, lds);
    ew<CM * CM / 4, 2>([&](int e) { return f4(dP)[e]; },
                       [&](int e, float4 x) {
                         const int i = (4 * e) / CM, j0 = (4 * e) % CM;
                         float* xs = reinterpret_cast<float*>(&x);
                         float4 y;
                         float* ys = reinterpret_cast<float*>(&y);
#pragma unroll
                         for (int q = 0; q < 4; ++q) {
                           const int j = j0 + q;
                           xs[q] = j <= i ? xs[q] : 0.f;
                           ys[q] = j <= i ? xs[q] * expf(v.g[i] - v.g[j]) : 0.f;
                         }
                         f4(dP)[e] = x;
                         f4(dPG)[e] = y;
                       });
    __syncthreads();
    // [X1; X2] = [dO; dU] S in one product (X2 = dU S = -dW)
    static_assert(sDU == sDO + 1 && sX2 == sX1 + 1, "dO, dU and X1, X2 adjacent");
    mm<2 * CM, D, D, false, false>(X1, D, dO, D, S, D, 1.f, nullptr, lds);
    // dq^ = diag(gamma) dO S + dPG K (the row dots q_i . (dO S)_i first)
    rowdot<D>(v.v1, X1, Q);   // q_i . (dO S)_i
    ew<CM * D / 4, 2>([&](int e) { return f4(X1)[e]; },
                      [&](int e, const float4& x) { f4(X1)[e] = v.gam[(4 * e) / D] * x; });
    __syncthreads();
    mm<CM, D, CM, false, false>(X1, D, dPG, CM, K, D, 1.f, X1, lds);
    // through the normalisation, into dq
    rowdot<D>(v.v2, X1, Q);   // q^ . dq^
    add_rows(dq, X1, Q, v.v2, v.rq, p.l2norm != 0);
    __syncthreads();
    // dW = -X2: T^T dW (X3), dT = dW (diag(b gamma) K)^T + dU (diag(b) V)^T (E1, one pass)
    mm<CM, D, CM, true, false>(X3, D, Tm, CM, X2, D, -1.f, nullptr, lds);
    mm2<CM, CM, D, false, true, D, false, true>(E1, CM, X2, D, BK, D, -1.f, dU, D, BV, D, 1.f, nullptr, lds);
    // T^T dU (X2)
    mm<CM, D, CM, true, false>(X2, D, Tm, CM, dU, D, 1.f, nullptr, lds);
    // dv = diag(b) T^T dU; row dots for db
    add_rows(dv, X2, nullptr, nullptr, v.b, false);
    rowdot<D>(v.v2, X2, V);   // (T^T dU)_i . v_i
    rowdot<D>(v.v3, X3, K);   // (T^T dW)_i . k_i
    // dA = strict_lower(-T^T dT T^T) (E1), via E2 = dT T^T
    mm<CM, CM, CM, false, true>(E2, CM, E1, CM, Tm, CM, 1.f, nullptr, lds);
    mm<CM, CM, CM, true, false>(E1, CM, Tm, CM, E2, CM, -1.f, nullptr, lds);
    // E2 = dKK = dA . (b_i Gam_ij); E (into dP) = dA . A + dP . P; E1 = dA . GK (row sums feed db)
    ew<CM * CM / 4, 2>(
        [&](int e) {
          F4x4 x;
          x.a = f4(E1)[e];
          x.b = f4(GK)[e];
          x.c = f4(dP)[e];
          x.d = f4(P)[e];
          return x;
        },
        [&](int e, F4x4 x) {
          const int i = (4 * e) / CM, j0 = (4 * e) % CM;
          float *e1 = reinterpret_cast<float*>(&x.a), *gk = reinterpret_cast<float*>(&x.b);
          float *dp = reinterpret_cast<float*>(&x.c), *pp = reinterpret_cast<float*>(&x.d);
          float4 y;
          float* e2 = reinterpret_cast<float*>(&y);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int j = j0 + q;
            const float dA = j < i ? e1[q] : 0.f;
            e2[q] = j < i ? dA * v.b[i] * expf(v.g[i] - v.g[j]) : 0.f;
            dp[q] = dA * v.b[i] * gk[q] + dp[q] * pp[q];
            e1[q] = dA * gk[q];
          }
          f4(E1)[e] = x.a;
          f4(E2)[e] = y;
          f4(dP)[e] = x.c;
        });
    __syncthreads();
    // gates: row sums minus column sums of E (in dP), row sums of dA . GK (in E1)
    {
      constexpr int LPR = CM / 4, RPP = kNT / LPR, PASSES = CM / RPP;   // 16 lanes per row, 4 passes
      const int c4 = threadIdx.x % LPR, r0 = threadIdx.x / LPR;
      float4 xe[PASSES], xg[PASSES];
#pragma unroll
      for (int q = 0; q < PASSES; ++q) {
        xe[q] = f4(dP)[(r0 + q * RPP) * LPR + c4];
        xg[q] = f4(E1)[(r0 + q * RPP) * LPR + c4];
      }
      float4 col = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int q = 0; q < PASSES; ++q) {
        float rs = xe[q].x + xe[q].y + xe[q].z + xe[q].w;
        float gs = xg[q].x + xg[q].y + xg[q].z + xg[q].w;
#pragma unroll
        for (int off = 1; off < LPR; off <<= 1) {
          rs += __shfl_xor(rs, off);
          gs += __shfl_xor(gs, off);
        }
        if (c4 == 0) {
          v.v4[r0 + q * RPP] = rs;
          v.gs[r0 + q * RPP] = gs;
        }
        col = col + xe[q];
      }
      // column partials: the lanes of a wave with the same c4 hold the same columns
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) {
        col.x += __shfl_xor(col.x, off);
        col.y += __shfl_xor(col.y, off);
        col.z += __shfl_xor(col.z, off);
        col.w += __shfl_xor(col.w, off);
      }
      if (lane < LPR) f4(v.cpart[wave])[c4] = col;
    }
    // <G, S>
    {
      float x = 0.f;
      ew<D * D / 4, 8>(
          [&](int e) {
            F4x2 y;
            y.a = f4(G)[e];
            y.b = f4(S)[e];
            return y;
          },
          [&](int, const F4x2& y) { x += dot4(y.a, y.b); });
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
      if (lane == 0) v.red[wave] = x;
    }
    __syncthreads();
    if (wave == 0) {
      const int i = lane;
      float cs = 0.f;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) cs += v.cpart[w][i];
      const float dbt = v.gam[i] * v.v3[i] + v.v2[i] + v.gs[i];
      if (i < n) db[g0 + size_t(i) * p.H] = dbt;
      float tsum = v.v0[i];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tsum += __shfl_xor(tsum, off);
      float GS = 0.f;
#pragma unroll
      for (int w = 0; w < kNT / 64; ++w) GS += v.red[w];
      float dg = v.v4[i] - cs + v.b[i] * v.gam[i] * v.v3[i] + v.gam[i] * v.v1[i] - v.v0[i];
      if (i == CM - 1) dg += v.gC * GS + tsum;
      // d(log a_t) = sum_{i >= t} dg_i
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(dg, off);
        if (i + off < 64) dg += y;
      }
      if (i < n) da[g0 + size_t(i) * p.H] = v.a[i] > 0.f ? dg / v.a[i] : 0.f;
    }
    // dk^ = De U G + diag(b gamma) T^T dW + dPG^T Q + (dKK + dKK^T) K; the
    // symmetric part of dKK into E1 (free after the gate sums)
    ew<CM * CM / 4, 4>(
        [&](int e) {
          const int i = (4 * e) / CM, j0 = (4 * e) % CM;
          F4x2 y;
          y.a = f4(E2)[e];
          y.b = make_float4(E2[(j0 + 0) * CM + i], E2[(j0 + 1) * CM + i], E2[(j0 + 2) * CM + i], E2[(j0 + 3) * CM + i]);
          return y;
        },
        [&](int e, const F4x2& y) { f4(E1)[e] = y.a + y.b; });
    mm<CM, D, D, false, false>(X1, D, U, D, G, D, 1.f, nullptr, lds);
    ew<CM * D / 4, 2>(
        [&](int e) {
          F4x2 y;
          y.a = f4(X1)[e];
          y.b = f4(X3)[e];
          return y;
        },
        [&](int e, const F4x2& y) {
          const int t = (4 * e) / D;
          f4(X1)[e] = v.De[t] * y.a + (v.b[t] * v.gam[t]) * y.b;
        });
    __syncthreads();
    mm2<CM, D, CM, true, false, CM, false, false>(X1, D, dPG, CM, Q, D, 1.f, E1, CM, K, D, 1.f, X1, lds);
    rowdot<D>(v.v2, X1, K);   // k^ . dk^
    add_rows(dk, X1, K, v.v2, v.rk, p.l2norm != 0);
    __syncthreads();
  }
}

// The two chains over chunks: S(c+1) = S(c) M_c + N_c forward from S(0) = S0
// (the start states, into Sst) and R(c-1) = R(c) M_c^T + X_c backward from
// R(n-1) = 0 (the adjoints reaching each chunk's end, into Rin; dS0 = R(-1)),
// both from the one stored M_c: the forward chain stages it k-major and reads
// it transposed, the backward one stages its rows as they are.
// A workgroup carries RW rows of the state through all chunks of one head and
// direction (grid (B*H, D/RW, 2)); each step is one RW x D by D x D product on
// split-bf16 MFMA, computed transposed, out^T = M^T S^T: the state stays in
// registers in the MFMA accumulator layout (lane = state row, values = 16
// state columns per 32 x 32 tile), which is also the B-operand layout of the
// next step once the reduction index is permuted the same way in both
// operands: B value i of lane l in k-step (tm, h) is column
// 32 tm + 16 h + 8 (i / 4) + 4 (l / 32) + i % 4, and the A operand reads those
// rows of M (k-major in LDS, two transposing reads of four rows each). Each
// step hands its tiles to the other waves through LDS (one 16-byte chunk per
// lane and half-tile); the matrices and addend rows are loaded into registers
// two steps ahead of their use.
template <int D>
constexpr int chain_threads() { return D == 128 ? 512 : 256; }   // two waves per SIMD at d = 128
// state rows per workgroup: 32 at d = 128 (four row blocks per head and
// direction; a step's matrix loads and record stores, not its products, set
// its time, so spreading the rows over more compute units shortens it)
template <int D>
constexpr int chain_rw() { return D == 128 ? 32 : D; }
// bf16 row pitch of the row-major staging: D + 4 puts consecutive rows two of
// the 64 four-byte banks apart, so the 32 rows of one 8-byte read are spread
// over all banks
template <int D>
constexpr int chain_row() { return D + 4; }
template <int D, int DIR>
__device__ __forceinline__ void chain_body(int n_chunks, const float* S0, const float* Am, const float* Um,
                                           const float* Xm, float* Sst, float* Rin, float* dS0, bf16* Mhi,
                                           bf16* Mlo, bf16x8_t* Xhi, bf16x8_t* Xlo) {
  constexpr int NTC = chain_threads<D>(), NW = NTC / 64;
  constexpr int RW = chain_rw<D>();                     // state rows per workgroup
  constexpr int TMO = D / 32, TN = RW / 32;            // output tiles: state columns x state rows
  constexpr int NTILE = TMO * TN, TPW = (NTILE + NW - 1) / NW;
  constexpr int PM = D * D / 4 / NTC;                  // float4 of the matrix per thread per step
  static_assert(PM * NTC * 4 == D * D, "the matrix splits evenly over the threads");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int bh = blockIdx.x, r0 = blockIdx.y * RW, dir = DIR;
  const size_t mat = size_t(D) * D;
  const size_t base = size_t(bh) * n_chunks * mat;
  const float* Mm = Am;
  const float* Nm = dir == 0 ? Um : Xm;
  float* rec = dir == 0 ? Sst : Rin;
  // this lane's place in tile u: state row r0 + 32 tn + l32, columns 32 tm + 8 j + 4 hl .. + 3
  auto tile_of = [&](int u, int& tm, int& tn) {
    const int t = wave + NW * u;
    tm = t / TN;
    tn = t % TN;
    return t < NTILE;
  };
  auto off4 = [&](int tm, int tn, int j) { return size_t(r0 + 32 * tn + l32) * D + 32 * tm + 8 * j + 4 * hl; };
  f32x16_t acc[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    int tm, tn;
    const bool own = tile_of(u, tm, tn);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (own && dir == 0 && S0) x = f4(S0 + size_t(bh) * mat)[off4(tm, tn, j) / 4];
      acc[u][4 * j] = x.x;
      acc[u][4 * j + 1] = x.y;
      acc[u][4 * j + 2] = x.z;
      acc[u][4 * j + 3] = x.w;
    }
  }
  // two register sets of a step's matrix and addend rows, each refilled two
  // steps ahead, so a load has two steps' products to arrive
  float4 nm0[PM], nm1[PM];
  float4 nn0[TPW][4], nn1[TPW][4];
  auto chunk_of = [&](int step) { return dir == 0 ? step : n_chunks - 1 - step; };
  auto fetch = [&](float4 (&nm)[PM], float4 (&nn)[TPW][4], int c) __attribute__((always_inline)) {
    const float4* M4 = f4(Mm + base + size_t(c) * mat);
#pragma unroll
    for (int i = 0; i < PM; ++i) nm[i] = M4[tid + i * NTC];
    const float* N = Nm + base + size_t(c) * mat;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      int tm, tn;
      const bool own = tile_of(u, tm, tn);
#pragma unroll
      for (int j = 0; j < 4; ++j) nn[u][j] = own ? f4(N)[off4(tm, tn, j) / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto body = [&](int step, float4 (&nm)[PM], float4 (&nn)[TPW][4]) __attribute__((always_inline)) {
    const int c = chunk_of(step);
    __syncthreads();   // the previous step's operand reads are done
    // record the state entering this step; hand it to the other waves as split operands
    float* rc = rec + base + size_t(c) * mat;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      int tm, tn;
      if (!tile_of(u, tm, tn)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f4(rc)[off4(tm, tn, j) / 4] = make_float4(acc[u][4 * j], acc[u][4 * j + 1], acc[u][4 * j + 2], acc[u][4 * j + 3]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8_t xh, xl;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float x = acc[u][8 * h + i];
          xh[i] = static_cast<bf16>(x);
          xl[i] = static_cast<bf16>(x - static_cast<float>(xh[i]));
        }
        Xhi[((tm * TN + tn) * 2 + h) * 64 + lane] = xh;
        Xlo[((tm * TN + tn) * 2 + h) * 64 + lane] = xl;
      }
    }
    // this step's matrix M, split: k-major for the forward chain (A = M^T, row
    // k of M holds its D columns), row-major rows of CRP for the backward one (A = M)
#pragma unroll
    for (int i = 0; i < PM; ++i) {
      const int e = tid + i * NTC;
      const int a = e / (D / 4), b4 = 4 * (e % (D / 4));
      const int o = DIR == 0 ? kmaj_off<D>(a, b4) : a * chain_row<D>() + b4;
      split_store4(Mhi + o, Mlo + o, nm[i]);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[u][4 * j] = nn[u][j].x;
        acc[u][4 * j + 1] = nn[u][j].y;
        acc[u][4 * j + 2] = nn[u][j].z;
        acc[u][4 * j + 3] = nn[u][j].w;
      }
    __syncthreads();
    // refill this set for two steps ahead (past the end it re-reads this step's chunk)
    fetch(nm, nn, chunk_of(step + 2 < n_chunks ? step + 2 : step));
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      int tm, tn;
      if (!tile_of(u, tm, tn)) continue;
      // out^T tile (rows: state columns 32 tm .., columns: state rows 32 tn ..)
      const int j16 = lane & 15, e = j16 >> 2, q = j16 & 3;
      const int col = 32 * tm + 16 * ((lane >> 4) & 1) + 4 * q;
#pragma unroll
      for (int km = 0; km < TMO; ++km)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x4_t a0, a1, b0, b1;
          if constexpr (DIR == 0) {
            const int kb = 32 * km + 16 * h + 4 * hl + e;
            a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Mhi + kmaj_off<D>(kb, col)));
            a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Mhi + kmaj_off<D>(kb + 8, col)));
            b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Mlo + kmaj_off<D>(kb, col)));
            b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(Mlo + kmaj_off<D>(kb + 8, col)));
          } else {
            // row 32 tm + l32 of M, reduction columns kb .. kb+3 and kb+8 .. kb+11
            const int o = (32 * tm + l32) * chain_row<D>() + 32 * km + 16 * h + 4 * hl;
            a0 = *reinterpret_cast<const bf16x4_t*>(Mhi + o);
            a1 = *reinterpret_cast<const bf16x4_t*>(Mhi + o + 8);
            b0 = *reinterpret_cast<const bf16x4_t*>(Mlo + o);
            b1 = *reinterpret_cast<const bf16x4_t*>(Mlo + o + 8);
          }
          const bf16x8_t ah = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          const bf16x8_t al = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          const bf16x8_t bh = Xhi[((km * TN + tn) * 2 + h) * 64 + lane];
          const bf16x8_t bl = Xlo[((km * TN + tn) * 2 + h) * 64 + lane];
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc[u], 0, 0, 0);
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc[u], 0, 0, 0);
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc[u], 0, 0, 0);
        }
    }
  };
  fetch(nm0, nn0, chunk_of(0));
  fetch(nm1, nn1, chunk_of(n_chunks > 1 ? 1 : 0));
  for (int step = 0; step < n_chunks; step += 2) {
    body(step, nm0, nn0);
    if (step + 1 < n_chunks) body(step + 1, nm1, nn1);
  }
  if (dir == 1 && dS0) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      int tm, tn;
      if (!tile_of(u, tm, tn)) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f4(dS0 + size_t(bh) * mat)[off4(tm, tn, j) / 4] =
            make_float4(acc[u][4 * j], acc[u][4 * j + 1], acc[u][4 * j + 2], acc[u][4 * j + 3]);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(chain_threads<D>())
gdn_bwd_chain_mfma(int n_chunks, const float* S0, const float* Am, const float* Um, const float* Xm, float* Sst,
                   float* Rin, float* dS0) {
  __shared__ __attribute__((aligned(16))) bf16 Mhi[D * chain_row<D>()], Mlo[D * chain_row<D>()];
  constexpr int NT2 = (D / 32) * (chain_rw<D>() / 32) * 2 * 64;
  __shared__ __attribute__((aligned(16))) bf16x8_t Xhi[NT2], Xlo[NT2];
  if (blockIdx.z == 0) chain_body<D, 0>(n_chunks, S0, Am, Um, Xm, Sst, Rin, dS0, Mhi, Mlo, Xhi, Xlo);
  else chain_body<D, 1>(n_chunks, S0, Am, Um, Xm, Sst, Rin, dS0, Mhi, Mlo, Xhi, Xlo);
}

template <typename Tin, typename Tg, int D>
hipError_t launch_t(const BwdArgs& x, int phase, hipStream_t st) {
  const Tg* g = static_cast<const Tg*>(x.d_mix);
  const dim3 grid(unsigned(x.n_slots < kBwdWorkgroups ? x.n_slots : kBwdWorkgroups));
  if (phase == 0)
    hipLaunchKernelGGL((gdn_bwd_mat_prep<Tin, Tg, D>), grid, dim3(kNT), 0, st, x.gdn, x.C, g, x.mix_w, x.slots,
                       x.slot_floats, x.Am, x.Um, x.Xm);
  else if (phase == 2)
    hipLaunchKernelGGL((gdn_bwd_chain_mfma<D>), dim3(unsigned(x.gdn.B * x.gdn.H), unsigned(D / chain_rw<D>()), 2),
                       dim3(chain_threads<D>()), 0, st, x.gdn.n_chunks, x.gdn.S0, x.Am, x.Um, x.Xm, x.Sst, x.Rin,
                       x.dS0);
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
