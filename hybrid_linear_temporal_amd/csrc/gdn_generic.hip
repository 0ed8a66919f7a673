// Generic gated-delta-rule kernels (fp32 arithmetic, d in {32, 64, 128},
// chunk C in {16, 32, 64}, float32 or bf16 inputs).
//
// The memory (Kairos related-work page, row A: the GatedDeltaNet state S_t
// with decay gate alpha_t; long-context page, section 06: erase the value
// stored under the current key, then write, with an overall forget gate):
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
// Chunked form (block-parallel inside a chunk, recurrent across chunks; the
// long-context page, sections 02 and 06, on chunkwise forms): with
// g_i = sum_{j<=i} log a_j over the chunk, gamma_i = exp(g_i),
//   A_ij = b_i exp(g_i - g_j) k_i.k_j (j < i),  T = (I + A)^-1,
//   W = T diag(b gamma) K,  U' = T diag(b) V,
//   U = U' - W S^T,  O = diag(gamma) Q S^T + [exp(g_i - g_j) q_i.k_j]_{j<=i} U,
//   S <- gamma_C S + U^T diag(gamma_C / gamma) K.
//
// Kernel 1 (gdn_prep): one workgroup per (chunk, head, batch row) computes
// the S-independent part of a chunk and writes it to the workspace record.
// Kernel 2 (gdn_chain): one workgroup per (16 rows of S, head, batch row)
// carries its rows of S through the chunks in order. Rows of S evolve
// independently, so the value dimension splits across workgroups.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerChain = 16;
constexpr float kL2Eps = 1e-6f;
constexpr float kLogAFloor = -80.f;

// Record of one chunk (floats): W | U' | Qg | Kd  ([C][D] each) | Aqk [C][C] | gamma_C
template <int D, int C>
struct Rec {
  static constexpr int W = 0, U = C * D, QG = 2 * C * D, KD = 3 * C * D, AQK = 4 * C * D,
                       GC = 4 * C * D + C * C;
};

template <typename Tin, int D, int C>
__global__ void __launch_bounds__(kThreads)
gdn_prep_generic(GdnParams p) {
  __shared__ float Ks[C][D];
  __shared__ float Xs[C][D];     // Q, later V
  __shared__ float M[C][C];      // A, then T = (I + A)^-1 in place (unit diagonal implicit)
  __shared__ float g[C], bb[C], rk[C], rq[C];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int tid = threadIdx.x;
  const long long t0 = (long long)chunk * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const Tin* q = static_cast<const Tin*>(p.q);
  const Tin* k = static_cast<const Tin*>(p.k);
  const Tin* v = static_cast<const Tin*>(p.v);
  const size_t HD = size_t(p.H) * D;
  const size_t base = (size_t(b) * p.L + t0) * HD + size_t(h) * D;
  const size_t gbase = (size_t(b) * p.L + t0) * p.H + h;

  for (int e = tid; e < C * D; e += kThreads) {
    const int i = e / D, col = e % D;
    const bool ok = i < n;
    Ks[i][col] = ok ? to_f32(k[base + i * HD + col]) : 0.f;
    Xs[i][col] = ok ? to_f32(q[base + i * HD + col]) : 0.f;
  }
  __syncthreads();
  if (tid < C) {
    float sk = 0.f, sq = 0.f;
    for (int col = 0; col < D; ++col) {
      sk += Ks[tid][col] * Ks[tid][col];
      sq += Xs[tid][col] * Xs[tid][col];
    }
    rk[tid] = p.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
    rq[tid] = p.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
  }
  if (tid == 0) {
    float acc = 0.f;
    for (int i = 0; i < C; ++i) {
      float la = 0.f, bi = 0.f;
      if (i < n) load_gates(p.a, p.b, gbase + size_t(i) * p.H, p.gate_logits, kLogAFloor, la, bi);
      acc += la;
      g[i] = acc;
      bb[i] = bi;
    }
  }
  __syncthreads();
  for (int e = tid; e < C * D; e += kThreads) {
    const int i = e / D, col = e % D;
    Ks[i][col] *= rk[i];
    Xs[i][col] *= rq[i];
  }
  __syncthreads();

  float* rec = reinterpret_cast<float*>(p.ws + (size_t(b * p.H + h) * p.n_chunks + chunk) * p.rec_bytes);
  using R = Rec<D, C>;
  // A (strictly lower) and Aqk (lower, inclusive)
  for (int e = tid; e < C * C; e += kThreads) {
    const int i = e / C, j = e % C;
    float kk = 0.f, qk = 0.f;
    if (j <= i) {
      for (int col = 0; col < D; ++col) {
        kk += Ks[i][col] * Ks[j][col];
        qk += Xs[i][col] * Ks[j][col];
      }
    }
    const float ratio = j <= i ? expf(g[i] - g[j]) : 0.f;
    M[i][j] = j < i ? bb[i] * ratio * kk : 0.f;
    rec[R::AQK + e] = ratio * qk;
  }
  // Q * gamma, K * gamma_C / gamma
  const float gl = g[C - 1];
  for (int e = tid; e < C * D; e += kThreads) {
    const int i = e / D, col = e % D;
    rec[R::QG + e] = expf(g[i]) * Xs[i][col];
    rec[R::KD + e] = expf(gl - g[i]) * Ks[i][col];
  }
  if (tid == 0) rec[R::GC] = expf(gl);
  __syncthreads();
  // forward substitution: T_i = e_i - sum_{j<i} A_ij T_j, row by row, in place
  for (int i = 1; i < C; ++i) {
    float t = 0.f;
    const int c = tid;
    if (c < i) {
      t = -M[i][c];
      for (int j = c + 1; j < i; ++j) t -= M[i][j] * M[j][c];
    }
    __syncthreads();
    if (c < i) M[i][c] = t;
    __syncthreads();
  }
  // V into Xs
  for (int e = tid; e < C * D; e += kThreads) {
    const int i = e / D, col = e % D;
    Xs[i][col] = i < n ? to_f32(v[base + i * HD + col]) : 0.f;
  }
  __syncthreads();
  // W = T diag(b gamma) K,  U' = T diag(b) V
  for (int e = tid; e < C * D; e += kThreads) {
    const int i = e / D, col = e % D;
    float w = bb[i] * expf(g[i]) * Ks[i][col];
    float u = bb[i] * Xs[i][col];
    for (int j = 0; j < i; ++j) {
      const float tij = M[i][j];
      w += tij * bb[j] * expf(g[j]) * Ks[j][col];
      u += tij * bb[j] * Xs[j][col];
    }
    rec[R::W + e] = w;
    rec[R::U + e] = u;
  }
}

template <typename Tout, int D, int C>
__global__ void __launch_bounds__(kThreads)
gdn_chain_generic(GdnParams p) {
  constexpr int NB = kRowsPerChain;
  __shared__ float Sb[NB][D];
  __shared__ float Ub[C][NB];
  using R = Rec<D, C>;

  const int v0 = blockIdx.x * NB, h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int tid = threadIdx.x;
  const size_t sbase = (size_t(b) * p.H + h) * D * D;
  for (int e = tid; e < NB * D; e += kThreads) {
    const int nn = e / D, col = e % D;
    Sb[nn][col] = p.S0 ? p.S0[sbase + size_t(v0 + nn) * D + col] : 0.f;
  }
  __syncthreads();
  Tout* o = static_cast<Tout*>(p.o);
  const size_t HD = size_t(p.H) * D;

  for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
    const float* rec =
        reinterpret_cast<const float*>(p.ws + (size_t(b * p.H + h) * p.n_chunks + chunk) * p.rec_bytes);
    const long long t0 = (long long)chunk * C;
    // U = U' - W S^T
    for (int e = tid; e < C * NB; e += kThreads) {
      const int i = e / NB, nn = e % NB;
      float u = rec[R::U + i * D + v0 + nn];
      for (int col = 0; col < D; ++col) u -= rec[R::W + i * D + col] * Sb[nn][col];
      Ub[i][nn] = u;
    }
    __syncthreads();
    // O = Qg S^T + Aqk U
    for (int e = tid; e < C * NB; e += kThreads) {
      const int i = e / NB, nn = e % NB;
      float acc = 0.f;
      for (int col = 0; col < D; ++col) acc += rec[R::QG + i * D + col] * Sb[nn][col];
      for (int j = 0; j <= i; ++j) acc += rec[R::AQK + i * C + j] * Ub[j][nn];
      const long long t = t0 + i;
      if (t < p.L) o[(size_t(b) * p.L + t) * HD + size_t(h) * D + v0 + nn] = from_f32<Tout>(acc);
    }
    __syncthreads();
    // S <- gamma_C S + U^T Kd
    const float gc = rec[R::GC];
    for (int e = tid; e < NB * D; e += kThreads) {
      const int nn = e / D, col = e % D;
      float s = gc * Sb[nn][col];
      for (int i = 0; i < C; ++i) s += Ub[i][nn] * rec[R::KD + i * D + col];
      Sb[nn][col] = s;
    }
    __syncthreads();
  }
  if (p.S_out) {
    for (int e = tid; e < NB * D; e += kThreads) {
      const int nn = e / D, col = e % D;
      p.S_out[sbase + size_t(v0 + nn) * D + col] = Sb[nn][col];
    }
  }
}

template <typename Tin, typename Tout, int D, int C>
hipError_t launch_t(const GdnParams& p, hipStream_t st) {
  hipLaunchKernelGGL((gdn_prep_generic<Tin, D, C>), dim3(p.n_chunks, p.H, p.B), dim3(kThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gdn_chain_generic<Tout, D, C>), dim3(D / kRowsPerChain, p.H, p.B), dim3(kThreads), 0,
                     st, p);
  return hipGetLastError();
}

template <typename Tin, typename Tout, int D>
hipError_t launch_c(const GdnParams& p, int C, hipStream_t st) {
  if (C == 16) return launch_t<Tin, Tout, D, 16>(p, st);
  if (C == 32) return launch_t<Tin, Tout, D, 32>(p, st);
  return launch_t<Tin, Tout, D, 64>(p, st);
}

template <typename Tin, typename Tout>
hipError_t launch_d(const GdnParams& p, int d, int C, hipStream_t st) {
  if (d == 32) return launch_c<Tin, Tout, 32>(p, C, st);
  if (d == 64) return launch_c<Tin, Tout, 64>(p, C, st);
  return launch_c<Tin, Tout, 128>(p, C, st);
}

}  // namespace

hipError_t launch_gdn_generic(const GdnParams& p, int d, int C, int in_dt, int out_dt, hipStream_t st) {
  if (in_dt == HLTA_F32) return launch_d<float, float>(p, d, C, st);
  if (out_dt == HLTA_BF16) return launch_d<bf16, bf16>(p, d, C, st);
  return launch_d<bf16, float>(p, d, C, st);
}

}  // namespace hlta
