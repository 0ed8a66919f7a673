// Backward of the operator (gradients for training): given dL/do_mix, the
// gradients of q, k, v, the gates, the mix weights and the start state. The
// branch gradients are do_i = w[h, i] * d_mix (the mix is linear). fp32
// kernels (any supported d and input dtype):
//
//  * softmax branches (exact attention, so its gradient is the textbook one;
//    long-context page, section 03 on tiled exact attention): a recompute pass
//    stores per query row the log2-sum-exp and D = do . o; a query-major pass
//    accumulates dq = s sum_k P (do . v_k - D) k; a key-major pass walks, for
//    each key frame, the query frames whose frame set holds it and
//    accumulates dv = sum_i P do_i and dk = s sum_i P (do_i . v - D_i) q_i;
//  * gated delta rule (Kairos related-work page, row A; long-context page,
//    section 06): with M_t = a_t (I - b_t k^ k^^T) the state obeys
//    S_t = S_{t-1} M_t + b_t v_t k^_t^T and its adjoint G_{t-1} = G_t M_t +
//    do_{t-1} q^_{t-1}^T. Per chunk of C tokens, in parallel, the transition
//    A_c (product of the M_t), the chunk's own state from zero U_c and its own
//    adjoint from zero X_c; then two short chains over chunks give every
//    chunk's start state and the adjoint reaching its end; then, per chunk in
//    parallel again, the states are recomputed token by token and the adjoint
//    carried back over the chunk, giving the token gradients (formulas at
//    gdn_bwd_tokens). Exact in fp32 (no approximation beyond rounding). The
//    prep gives each wave 16 rows of one matrix (rows evolve independently);
//    the token pass keeps S and G as per-thread (d/16) x (d/16) blocks;
//  * mix weights: dw[h, i] = <d_mix, o_i> over the stored branch outputs.
// With bf16 inputs and outputs, d = 128 and P >= 64 the softmax branches run
// on the bf16 MFMA kernels of attn_bwd_mfma.hip instead.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;
constexpr float kL2Eps = 1e-6f;

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

// Block layout: thread t owns rows 16-block t/16 and columns 16-block t%16 of
// a d x d matrix, BS = d/16 each. Matrix-vector products: each thread writes
// the partial sums of its block to LDS and, after one barrier, the 16 partials
// of an entry are added in a fixed order; up to four products share a round.
// Scalar sums: wave reduction, then the four wave partials from LDS.
template <int D>
struct GdnBlock {
  static constexpr int BS = D / 16;
  float red[4][16][D];   // partial sums of up to four matrix-vector products
  float vec[12][D];      // vectors of the current token
  float wsum[8][8][4];   // wave partials of up to 8 sums, 8 slots
};

// partial sums of y = M x (kRows) or y = M^T x into red[slot]
template <int D, bool kRows>
__device__ __forceinline__ void mv_part(GdnBlock<D>& sm, const float (&M)[D / 16][D / 16], const float* x, int slot) {
  constexpr int BS = D / 16;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int a = 0; a < BS; ++a) {
    float s = 0.f;
#pragma unroll
    for (int bb = 0; bb < BS; ++bb) s += kRows ? M[a][bb] * x[tc * BS + bb] : M[bb][a] * x[tr * BS + bb];
    if (kRows) sm.red[slot][tc][tr * BS + a] = s;
    else sm.red[slot][tr][tc * BS + a] = s;
  }
}
// vec[y[slot]] = f[slot] * (sum of the partials of slot), slots 0 .. n-1 (after a barrier)
template <int D>
__device__ __forceinline__ void mv_finish(GdnBlock<D>& sm, int n, const int (&y)[4], const float (&f)[4]) {
  for (int e = threadIdx.x; e < n * D; e += kThreads) {
    const int slot = e / D, i = e % D;
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) s += sm.red[slot][g][i];
    sm.vec[y[slot]][i] = s * f[slot];
  }
}

// N sums of one value per thread; every thread gets the totals. Slot picks a
// private LDS area (a slot is reused only after further barriers).
template <int D, int N>
__device__ __forceinline__ void sum_n(GdnBlock<D>& sm, float (&x)[N], int slot) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float v = x[j];
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    x[j] = v;
  }
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int j = 0; j < N; ++j) sm.wsum[slot][j][threadIdx.x >> 6] = x[j];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < N; ++j) x[j] = sm.wsum[slot][j][0] + sm.wsum[slot][j][1] + sm.wsum[slot][j][2] + sm.wsum[slot][j][3];
}

__device__ __forceinline__ float l2n(float n2, bool on) { return on ? sqrtf(n2 + kL2Eps) : 1.f; }

// One token of the memory on S (held in blocks): vec[0] = k and vec[1] = v
// are in LDS (written before a barrier); applies S <- a (S - b u k^^T)
// (+ b v k^^T when with_v) with k^ = k / n(k) and u = S k^ (S k and |k|^2 in
// one round).
template <int D>
__device__ __forceinline__ void fwd_token(GdnBlock<D>& sm, float (&S)[D / 16][D / 16], float at, float bt, bool l2,
                                          bool with_v) {
  constexpr int BS = D / 16;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  mv_part<D, true>(sm, S, sm.vec[0], 0);
  float n2[1] = {threadIdx.x < D ? sm.vec[0][threadIdx.x] * sm.vec[0][threadIdx.x] : 0.f};
  sum_n<D, 1>(sm, n2, 0);   // its barrier also completes the partials
  const float inv = 1.f / l2n(n2[0], l2);
  mv_finish<D>(sm, 1, {3, 0, 0, 0}, {inv, 1.f, 1.f, 1.f});   // u = S k / n
  __syncthreads();
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const float kj = sm.vec[0][tc * BS + j] * inv;
      const float vt = with_v ? bt * sm.vec[1][tr * BS + i] * kj : 0.f;
      S[i][j] = at * (S[i][j] - bt * sm.vec[3][tr * BS + i] * kj) + vt;
    }
  __syncthreads();
}

template <int D>
__device__ __forceinline__ void load_mat(float (&M)[D / 16][D / 16], const float* src) {
  constexpr int BS = D / 16;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) M[i][j] = src ? src[size_t(tr * BS + i) * D + tc * BS + j] : 0.f;
}
template <int D>
__device__ __forceinline__ void store_mat(float* dst, const float (&M)[D / 16][D / 16]) {
  constexpr int BS = D / 16;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
#pragma unroll
  for (int i = 0; i < BS; ++i)
#pragma unroll
    for (int j = 0; j < BS; ++j) dst[size_t(tr * BS + i) * D + tc * BS + j] = M[i][j];
}

// CPL consecutive values of a [.., D] row (bf16 or fp32) as floats
template <int CPL>
__device__ __forceinline__ void load_cols(const bf16* p, float (&x)[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL; i += 8) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + i);
    const bf16* e = reinterpret_cast<const bf16*>(&u);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[i + j] = static_cast<float>(e[j]);
  }
}
template <int CPL>
__device__ __forceinline__ void load_cols(const float* p, float (&x)[CPL]) {
#pragma unroll
  for (int i = 0; i < CPL; i += 4) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + i);
    const float* e = reinterpret_cast<const float*>(&u);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[i + j] = e[j];
  }
}

// sum over the 4 lanes of a row (lanes 4r .. 4r+3)
__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Chunk c of head (b, h) covers tokens [c*C, min(L, (c+1)*C)). With
// M_t = a_t (I - b_t k^_t k^_t^T) (symmetric), per chunk:
//   kWhat 0: A_c = M_s M_{s+1} .. M_e            (S_end = S_start A_c + U_c)
//   kWhat 1: U_c = the chunk's own state from S = 0
//   kWhat 2: X_c = sum_t do_t q^_t^T M_t M_{t-1} .. M_s
//            (the chunk's own adjoint carried to its start; G = dL/dS)
// Rows of all three evolve independently (row i of A M_t is a (a_i - b
// (a_i . k^) k^)), so each wave owns 16 rows: lane = (row lane/4, quarter
// lane%4 of the columns), row dot products by two lane shuffles, no barrier
// inside the token loop. The workgroup (4 waves, 64 rows) first stages the
// chunk's k (and q), the rows' v (or d_mix) and the gates in LDS, so a token
// costs LDS reads only. grid (B*H*n_chunks, ceil(D/64)).
constexpr int kMaxChunk = 64;
template <typename Tin, typename Tg, int D, int kWhat>
__global__ void __launch_bounds__(kThreads)
gdn_bwd_prep(GdnParams p, int C, const Tg* d_mix, const float* mix_w, float* out, float* AmT) {
  constexpr int CPL = D / 4;
  __shared__ __attribute__((aligned(16))) Tin kS[kMaxChunk][D];
  __shared__ __attribute__((aligned(16))) Tin qS[kWhat == 2 ? kMaxChunk : 1][D];
  __shared__ float xS[kWhat >= 1 ? kMaxChunk : 1][64];
  __shared__ float aS[kMaxChunk], bS[kMaxChunk];
  const long long job = blockIdx.x;
  const int c = int(job % p.n_chunks), bh = int(job / p.n_chunks), b = bh / p.H, h = bh % p.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane >> 2, c0 = (lane & 3) * CPL;
  const int R0 = blockIdx.y * 64;
  const int row = R0 + wave * 16 + r;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const long long t0 = (long long)c * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const bool l2 = p.l2norm != 0;
  const size_t tok0 = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
  const size_t g0 = (size_t(b) * p.L + t0) * p.H + h;
  for (int e = threadIdx.x; e < n * D; e += kThreads) {
    const int t = e / D, col = e % D;
    kS[t][col] = k[tok0 + size_t(t) * HD + col];
    if constexpr (kWhat == 2) qS[t][col] = q[tok0 + size_t(t) * HD + col];
  }
  if constexpr (kWhat >= 1) {
    const float w2 = mix_w[3 * h + 2];
    for (int e = threadIdx.x; e < n * 64; e += kThreads) {
      const int t = e / 64, rr = R0 + e % 64;
      float x = 0.f;
      if (rr < D) x = kWhat == 1 ? ld(v, tok0 + size_t(t) * HD + rr) : w2 * ld(d_mix, tok0 + size_t(t) * HD + rr);
      xS[t][e % 64] = x;
    }
  }
  if (threadIdx.x < n) {
    aS[threadIdx.x] = p.a[g0 + size_t(threadIdx.x) * p.H];
    bS[threadIdx.x] = p.b[g0 + size_t(threadIdx.x) * p.H];
  }
  __syncthreads();
  if (R0 + wave * 16 >= D) return;   // d = 32: two waves have no rows
  float M[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) M[j] = (kWhat == 0 && c0 + j == row) ? 1.f : 0.f;
  for (int i = 0; i < n; ++i) {
    const int s = kWhat == 2 ? n - 1 - i : i;
    float kx[CPL];
    load_cols<CPL>(&kS[s][c0], kx);
    const float at = aS[s], bt = bS[s];
    float k2 = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) k2 += kx[j] * kx[j];
    const float ik = 1.f / l2n(quad_sum(k2), l2);
    if constexpr (kWhat == 2) {   // M <- M + do q^^T
      float qx[CPL];
      load_cols<CPL>(&qS[s][c0], qx);
      float q2 = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) q2 += qx[j] * qx[j];
      const float f = xS[s][wave * 16 + r] / l2n(quad_sum(q2), l2);
#pragma unroll
      for (int j = 0; j < CPL; ++j) M[j] += f * qx[j];
    }
    float u = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) u += M[j] * kx[j];
    u = quad_sum(u) * ik;
    // M <- a (M - b u k^^T) (+ b v k^^T for the own state)
    const float cu = at * bt * u * ik;
    const float cv = kWhat == 1 ? bt * xS[s][wave * 16 + r] * ik : 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) M[j] = at * M[j] + (cv - cu) * kx[j];
  }
  float* dst = out + size_t(job) * D * D + size_t(row) * D + c0;
#pragma unroll
  for (int j = 0; j < CPL; j += 4) *reinterpret_cast<float4*>(dst + j) = make_float4(M[j], M[j + 1], M[j + 2], M[j + 3]);
  if constexpr (kWhat == 0) {   // A^T too, so both chains run the same row-times-matrix product
    float* t = AmT + size_t(job) * D * D + row;
#pragma unroll
    for (int j = 0; j < CPL; ++j) t[size_t(c0 + j) * D] = M[j];
  }
}

// The two chains over chunks, rows of the state split over workgroups (rows
// evolve independently: row i of S A + U only needs row i of S and U):
//   dir 0: S_start(0) = S0, S_start(c+1) = S_start(c) A_c + U_c
//   dir 1: R(N-1) = 0,      R(c-1) = R(c) A_c^T + X_c, dS0 = R(-1)
// R(c) is the adjoint reaching the end of chunk c from later tokens. The
// matrix (A_c, or A_c^T as the prep stored it) is staged in LDS rows padded
// to keep 16-byte alignment; a thread owns one row of the group and CPT
// consecutive columns, read as float4s, and the row itself is read four
// values at a time. The next step's matrix and U/X rows are loaded into
// registers while the current step computes (the chain is latency-bound: one
// dependent 16 x d by d x d product per chunk). grid (B*H, D/16, 2).
constexpr int kChainRows = 16;
typedef float v4f __attribute__((ext_vector_type(4)));
template <int D>
__global__ void __launch_bounds__(kThreads)
gdn_bwd_chain(int n_chunks, const float* S0, const float* Am, const float* AmT, const float* Um, const float* Xm,
              float* Sst, float* Rin, float* dS0) {
  constexpr int DP = D + 4;                        // padded row (floats), keeps float4 alignment
  __shared__ __attribute__((aligned(16))) float As[D * DP];
  __shared__ __attribute__((aligned(16))) float rows[kChainRows][D];
  constexpr int CPT = D * kChainRows / kThreads;   // columns per thread: 8 (d = 128), 4 (64), 2 (32)
  constexpr int PER = D * D / 4 / kThreads;        // float4 of the matrix per thread per step
  const int bh = blockIdx.x, r0 = blockIdx.y * kChainRows, dir = blockIdx.z;
  const int r = threadIdx.x / (D / CPT), j0 = (threadIdx.x % (D / CPT)) * CPT;
  const size_t mat = size_t(D) * D;
  const size_t base = size_t(bh) * n_chunks * mat;
  const float* Mm = dir == 0 ? Am : AmT;
  const float* Bm = dir == 0 ? Um : Xm;
#pragma unroll
  for (int jj = 0; jj < CPT; ++jj)
    rows[r][j0 + jj] = (dir == 0 && S0) ? S0[size_t(bh) * mat + size_t(r0 + r) * D + j0 + jj] : 0.f;
  v4f na[PER];
  float nb[CPT];
  auto fetch = [&](int c) __attribute__((always_inline)) {
    const v4f* A4 = reinterpret_cast<const v4f*>(Mm + base + size_t(c) * mat);
#pragma unroll
    for (int i = 0; i < PER; ++i) na[i] = A4[threadIdx.x + i * kThreads];
    const float* add = Bm + base + size_t(c) * mat + size_t(r0 + r) * D + j0;
#pragma unroll
    for (int jj = 0; jj < CPT; ++jj) nb[jj] = add[jj];
  };
  fetch(dir == 0 ? 0 : n_chunks - 1);
  for (int step = 0; step < n_chunks; ++step) {
    const int c = dir == 0 ? step : n_chunks - 1 - step;
    __syncthreads();   // the previous step no longer reads As or rows
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (threadIdx.x + i * kThreads) * 4;
      *reinterpret_cast<v4f*>(&As[(e / D) * DP + e % D]) = na[i];
    }
    float out[CPT];
#pragma unroll
    for (int jj = 0; jj < CPT; ++jj) out[jj] = nb[jj];
    // unconditional (the last step re-reads its own chunk) so the prefetch buffer stays in registers
    fetch(dir == 0 ? (c + 1 < n_chunks ? c + 1 : c) : (c > 0 ? c - 1 : 0));
    __syncthreads();
    float* rec = (dir == 0 ? Sst : Rin) + base + size_t(c) * mat + size_t(r0 + r) * D + j0;
#pragma unroll
    for (int jj = 0; jj < CPT; ++jj) rec[jj] = rows[r][j0 + jj];
    // out += x * (row k of the matrix), CPT consecutive columns from j0
    auto axpy = [&](float x, int k) __attribute__((always_inline)) {
      const float* arow = &As[k * DP + j0];
      if constexpr (CPT >= 4) {
#pragma unroll
        for (int j4 = 0; j4 < CPT; j4 += 4) {
          const v4f a4 = *reinterpret_cast<const v4f*>(arow + j4);
          out[j4] += x * a4.x;
          out[j4 + 1] += x * a4.y;
          out[j4 + 2] += x * a4.z;
          out[j4 + 3] += x * a4.w;
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < CPT; ++jj) out[jj] += x * arow[jj];
      }
    };
#pragma unroll 4
    for (int k4 = 0; k4 < D; k4 += 4) {
      const v4f x = *reinterpret_cast<const v4f*>(&rows[r][k4]);
      axpy(x.x, k4);
      axpy(x.y, k4 + 1);
      axpy(x.z, k4 + 2);
      axpy(x.w, k4 + 3);
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < CPT; ++jj) rows[r][j0 + jj] = out[jj];
  }
  if (dir == 1 && dS0) {
#pragma unroll
    for (int jj = 0; jj < CPT; ++jj) dS0[size_t(bh) * mat + size_t(r0 + r) * D + j0 + jj] = rows[r][j0 + jj];
  }
}

// Gradients of one chunk's tokens from its start state S_start(c) and the
// adjoint R(c) reaching its end: the chunk's states are recomputed into this
// workgroup's slot, then the adjoint is carried backwards token by token.
// With G = dL/dS_t (it gains do_t q^^T at token t), u = S_{t-1} k^:
//   dq^ = S_t^T do_t = a (S_{t-1}^T do - b k^ (u . do)) + b k^ (v . do)
//   da = <G, S_{t-1}> - b (u . G k^),  dv = b G k^,
//   db = v . G k^ - a (u . G k^),
//   dk^ = b G^T v - a b (S_{t-1}^T G k^ + G^T u),
//   G <- a (G - b (G k^) k^^T)  (dL/dS_{t-1}),
// and dx = dx^/n - x (x . dx^)/n^3 through the L2 normalisation.
// Persistent: workgroup i takes jobs i, i + grid, ... (job = (b*H + h)*N + c).
template <typename Tin, typename Tg, int D>
__global__ void __launch_bounds__(kThreads)
gdn_bwd_tokens(GdnParams p, int C, const float* Sst, const float* Rin, float* slots, const Tg* d_mix,
               const float* mix_w, float* dq, float* dk, float* dv, float* da, float* db) {
  constexpr int BS = D / 16;
  __shared__ GdnBlock<D> sm;
  const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const size_t mat = size_t(D) * D;
  float* cb = slots + size_t(blockIdx.x) * C * mat;
  const long long jobs = (long long)p.B * p.H * p.n_chunks;
  const bool l2 = p.l2norm != 0;
  auto blk = [&](int i, int j) { return size_t(tr * BS + i) * D + tc * BS + j; };
  for (long long job = blockIdx.x; job < jobs; job += gridDim.x) {
    const int c = int(job % p.n_chunks), bh = int(job / p.n_chunks), b = bh / p.H, h = bh % p.H;
    const float w2 = mix_w[3 * h + 2];
    const long long t0 = (long long)c * C;
    const int n = int(p.L - t0 < C ? p.L - t0 : C);
    float S[BS][BS], G[BS][BS];
    load_mat<D>(S, Sst + size_t(job) * mat);
    // the next token's vectors and gates are loaded while the current one computes
    const size_t tok0 = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
    const size_t g0 = (size_t(b) * p.L + t0) * p.H + h;
    const int e = threadIdx.x < D ? threadIdx.x : 0;
    float xk = ld(k, tok0 + e), xv = ld(v, tok0 + e), xa = p.a[g0], xb = p.b[g0];
    for (int s = 0; s < n; ++s) {
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) cb[size_t(s) * mat + blk(i, j)] = S[i][j];
      if (threadIdx.x < D) {
        sm.vec[0][threadIdx.x] = xk;
        sm.vec[1][threadIdx.x] = xv;
      }
      const float at = xa, bt = xb;
      __syncthreads();
      if (s + 1 < n) {
        xk = ld(k, tok0 + size_t(s + 1) * HD + e);
        xv = ld(v, tok0 + size_t(s + 1) * HD + e);
        xa = p.a[g0 + size_t(s + 1) * p.H];
        xb = p.b[g0 + size_t(s + 1) * p.H];
      }
      fwd_token(sm, S, at, bt, l2, true);
    }
    load_mat<D>(G, Rin + size_t(job) * mat);
    float xq = 0.f, xd = 0.f;
    {
      const size_t o = tok0 + size_t(n - 1) * HD + e;
      xk = ld(k, o), xv = ld(v, o), xq = ld(q, o), xd = w2 * ld(d_mix, o);
      xa = p.a[g0 + size_t(n - 1) * p.H], xb = p.b[g0 + size_t(n - 1) * p.H];
    }
    for (int s = n - 1; s >= 0; --s) {
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) S[i][j] = cb[size_t(s) * mat + blk(i, j)];   // S_{t-1}
      const long long t = t0 + s;
      const size_t tok = (size_t(b) * p.L + t) * HD + size_t(h) * D;
      const size_t g = (size_t(b) * p.L + t) * p.H + h;
      const float at = xa, bt = xb;
      // vec: 0 k, 1 v, 3 q, 5 do, 6 u = S k^, 7 S^T do, 8 G k^, 9 G^T v, 10 G^T u, 11 S^T G k^
      // (k^ = k ik and q^ = q iq are formed on the fly)
      if (threadIdx.x < D) {
        sm.vec[0][threadIdx.x] = xk;
        sm.vec[1][threadIdx.x] = xv;
        sm.vec[3][threadIdx.x] = xq;
        sm.vec[5][threadIdx.x] = xd;
      }
      __syncthreads();
      if (s > 0) {
        const size_t o = tok0 + size_t(s - 1) * HD + e;
        xk = ld(k, o), xv = ld(v, o), xq = ld(q, o), xd = w2 * ld(d_mix, o);
        xa = p.a[g0 + size_t(s - 1) * p.H], xb = p.b[g0 + size_t(s - 1) * p.H];
      }
      float n2[2] = {0.f, 0.f};
      if (threadIdx.x < D) {
        n2[0] = sm.vec[0][threadIdx.x] * sm.vec[0][threadIdx.x];
        n2[1] = sm.vec[3][threadIdx.x] * sm.vec[3][threadIdx.x];
      }
      sum_n<D, 2>(sm, n2, 0);
      const float ik = 1.f / l2n(n2[0], l2), iq = 1.f / l2n(n2[1], l2);
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) G[i][j] += sm.vec[5][tr * BS + i] * sm.vec[3][tc * BS + j] * iq;
      mv_part<D, true>(sm, S, sm.vec[0], 0);    // S k
      mv_part<D, false>(sm, S, sm.vec[5], 1);   // S^T do
      mv_part<D, true>(sm, G, sm.vec[0], 2);    // G k
      mv_part<D, false>(sm, G, sm.vec[1], 3);   // G^T v
      __syncthreads();
      mv_finish<D>(sm, 4, {6, 7, 8, 9}, {ik, 1.f, ik, 1.f});
      __syncthreads();
      mv_part<D, false>(sm, G, sm.vec[6], 0);   // G^T u
      mv_part<D, false>(sm, S, sm.vec[8], 1);   // S^T G k^
      float sc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};  // <G, S>, u.do, v.do, u.Gk^, v.Gk^
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j) sc[0] += G[i][j] * S[i][j];
      if (threadIdx.x < D) {
        const int i = threadIdx.x;
        sc[1] = sm.vec[6][i] * sm.vec[5][i];
        sc[2] = sm.vec[1][i] * sm.vec[5][i];
        sc[3] = sm.vec[6][i] * sm.vec[8][i];
        sc[4] = sm.vec[1][i] * sm.vec[8][i];
      }
      sum_n<D, 5>(sm, sc, 1);   // its barrier also completes the second round's partials
      mv_finish<D>(sm, 2, {10, 11, 0, 0}, {1.f, 1.f, 1.f, 1.f});
      __syncthreads();
      const float GS = sc[0], udo = sc[1], vdo = sc[2], uGk = sc[3], vGk = sc[4];
      if (threadIdx.x == 0) {
        da[g] = GS - bt * uGk;
        db[g] = vGk - at * uGk;
      }
      float dqh = 0.f, dkh = 0.f, qi = 0.f, ki = 0.f;
      float d2[2] = {0.f, 0.f};
      if (threadIdx.x < D) {
        const int i = threadIdx.x;
        ki = sm.vec[0][i];
        qi = sm.vec[3][i];
        const float kh = ki * ik;
        dqh = at * (sm.vec[7][i] - bt * kh * udo) + bt * kh * vdo;
        dkh = bt * sm.vec[9][i] - at * bt * (sm.vec[11][i] + sm.vec[10][i]);
        dv[tok + i] += bt * sm.vec[8][i];
        d2[0] = qi * dqh;
        d2[1] = ki * dkh;
      }
      sum_n<D, 2>(sm, d2, 2);
      if (threadIdx.x < D) {
        const int i = threadIdx.x;
        dq[tok + i] += l2 ? dqh * iq - qi * d2[0] * iq * iq * iq : dqh;
        dk[tok + i] += l2 ? dkh * ik - ki * d2[1] * ik * ik * ik : dkh;
      }
#pragma unroll
      for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j)
          G[i][j] = at * (G[i][j] - bt * sm.vec[8][tr * BS + i] * sm.vec[0][tc * BS + j] * ik);
      __syncthreads();
    }
  }
}

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
    const hipError_t e = launch_attn_bwd_mfma(p, x.d_mix, x.o_swa, x.o_dswa, x.mix_w, x.lse2, x.dsum, x.dq, x.dk,
                                              x.dv, x.scale, st);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((attn_bwd_stats<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum);
    hipLaunchKernelGGL((attn_bwd_dq<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum,
                       x.dq, x.scale);
    hipLaunchKernelGGL((attn_bwd_dkdv<Tin, Tg, D>), grid, dim3(kThreads), 0, st, p, g, x.mix_w, x.lse2, x.dsum,
                       x.dk, x.dv, x.scale);
  }
  const unsigned heads = unsigned(x.gdn.B * x.gdn.H);
  const unsigned jobs = heads * unsigned(x.gdn.n_chunks);
  const dim3 pgrid(jobs, (D + 63) / 64);
  hipLaunchKernelGGL((gdn_bwd_prep<Tin, Tg, D, 0>), pgrid, dim3(kThreads), 0, st, x.gdn, x.C, g, x.mix_w, x.Am, x.AmT);
  hipLaunchKernelGGL((gdn_bwd_prep<Tin, Tg, D, 1>), pgrid, dim3(kThreads), 0, st, x.gdn, x.C, g, x.mix_w, x.Um, x.AmT);
  hipLaunchKernelGGL((gdn_bwd_prep<Tin, Tg, D, 2>), pgrid, dim3(kThreads), 0, st, x.gdn, x.C, g, x.mix_w, x.Xm, x.AmT);
  hipLaunchKernelGGL((gdn_bwd_chain<D>), dim3(heads, D / kChainRows, 2), dim3(kThreads), 0, st, x.gdn.n_chunks,
                     x.gdn.S0, x.Am, x.AmT, x.Um, x.Xm, x.Sst, x.Rin, x.dS0);
  hipLaunchKernelGGL((gdn_bwd_tokens<Tin, Tg, D>), dim3(unsigned(x.n_slots)), dim3(kThreads), 0, st, x.gdn, x.C,
                     x.Sst, x.Rin, x.slots, g, x.mix_w, x.dq, x.dk, x.dv, x.da, x.db);
  return hipGetLastError();
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
