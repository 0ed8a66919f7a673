// Gated delta rule with bf16 MFMA on gfx950 (bf16 inputs, d = 128, chunk 64).
//
// The memory (Kairos related-work page, row A: the GatedDeltaNet state S_t
// with decay gate alpha_t; long-context page, section 06: erase what the
// current key stores, then write, under an overall forget gate):
//   S_t = a_t S_{t-1} (I - b_t k^_t k^_t^T) + b_t v_t k^_t^T,  o_t = S_t q^_t,
// with q^, k^ the L2-normalised q, k. Chunked form (block-parallel inside a
// chunk, recurrent across chunks; long-context page, sections 02 and 06): with
// g_i = sum_{j<=i} log a_j, gamma_i = exp(g_i) inside a chunk,
//   A_ij = b_i exp(g_i - g_j) k^_i.k^_j (j < i),  T = (I + A)^-1,
//   W = T diag(b gamma) K^,  U' = T diag(b) V,
//   U = U' - W S^T,  O = diag(gamma) Q^ S^T + [exp(g_i - g_j) q^_i.k^_j]_{j<=i} U,
//   S <- gamma_C S + U^T diag(gamma_C / gamma) K^.
//
// Kernel 1, gdn_prep_mfma: one workgroup per (chunk, head, batch row), fully
// parallel, two per CU. Gram matrices K K^T and Q K^T on raw bf16 inputs
// (exact products, fp32 sums) with the norms and gates applied in fp32; T by
// blocked forward substitution in fp32 (16x16 diagonal blocks per wave, then
// the off-diagonal blocks level by level); W^T and U' on MFMA with the raw K,
// V read transposed from LDS (ds_read_b64_tr_b16). Writes one record per chunk.
//
// Kernel 2, gdn_chain_mfma: one workgroup per (16 value channels, head, batch
// row), chunks in order; the 8 workgroups of a head sit on one XCD and share
// its L2. Four waves, one per SIMD: the state wave keeps the slice of S^T
// (128 x 16, fp32) in MFMA accumulator layout for the whole sequence and runs
// U = U' - W S^T and the state update; the output wave recomputes U from the
// same operands and writes O; the loader wave streams the next chunk's
// operands into the second LDS buffer; the prefetch wave pulls later chunks
// into L2. The bf16 copy of S^T, published in LDS by the state wave, is the B
// operand of W S^T and the A operand of S q^T directly, because the 16x16x32
// A and B layouts coincide and the reduction (d_k) index of an MFMA may be
// permuted as long as both operands agree; the other operands are read from
// LDS in that permuted order. The same holds for U (C layout) as operand of
// the state update and of U^T Aqk^T, so S and U are never transposed.
#include "hlta_device.h"
#include "hlta_internal.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int D = 128;
constexpr int C = 64;
constexpr int NT = 256;
constexpr float kL2Eps = 1e-6f;
constexpr float kLogAFloor = -80.f;
using R = GdnMfmaRec;
static_assert(R::C == C && R::D == D, "record layout");

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Transposed LDS read (gfx950): inside each group of 16 lanes, lane j gets
// element j%4 of the 4-element rows addressed by lanes 4e + j/4, e = 0..3.
__device__ __forceinline__ bf16x4 ld_tr(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// direct global -> LDS loads, padded-tile helpers
__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Source offset of chunk slot P of a padded tile (row P / pitch, chunk P % pitch).
__device__ __forceinline__ unsigned slot_offset(int P, int pitch_chunks, int src_chunks, int src_row_bytes,
                                                int clamp_row) {
  int row = P / pitch_chunks, ch = P - row * pitch_chunks;
  if (ch >= src_chunks) ch = src_chunks - 1;
  if (row > clamp_row) row = clamp_row;
  return unsigned(row) * unsigned(src_row_bytes) + unsigned(ch) * 16u;
}

// 4 consecutive bf16 at (row, col) of a padded tile
template <int PC>
__device__ __forceinline__ bf16x4 ld4p(const uint4* t, int row, int col) {
  return *reinterpret_cast<const bf16x4*>(reinterpret_cast<const char*>(t) + row * (PC * 16) + col * 2);
}
template <int PC>
__device__ __forceinline__ bf16x4 ld4p_tr(const uint4* t, int row, int col) {
  return ld_tr(reinterpret_cast<const bf16*>(reinterpret_cast<const char*>(t) + row * (PC * 16) + col * 2));
}

__device__ __forceinline__ unsigned tok_offset(unsigned off256, int last_row, unsigned tok_bytes) {
  unsigned row = off256 >> 8;
  if (row > unsigned(last_row)) row = unsigned(last_row);
  return row * tok_bytes + (off256 & 255u);
}

// ---------------------------------------------------------------------------
// kernel 1: per-chunk preparation
// ---------------------------------------------------------------------------

// LDS of one chunk (76 KB, two workgroups per CU). K, Q, V tiles have 272-byte
// rows (17 chunk slots, filled by direct loads); the Q tile is reused for A
// after the Gram products, and the T region first stages Aqk, then holds T,
// then the bf16 T' = T diag(b gamma / ||k||) and T'' = T diag(b).
constexpr int PQ = 17;           // chunk slots per K/Q/V row
constexpr int AP = 68;           // fp32 pitch of A and T
constexpr int TP = 68;           // bf16 pitch of T' and T''
constexpr int TILE_BYTES = C * PQ * 16;
static_assert(C * AP * 4 == TILE_BYTES, "A and T fill one tile region");
struct PrepSmem {
  uint4 K[C * PQ];
  uint4 V[C * PQ];
  uint4 QA[C * PQ];            // Q tile, then A (fp32 [C][AP])
  uint4 TT[C * PQ];            // Aqk staging (bf16 [C][72]), then T (fp32 [C][AP]), then T', T''
  float X[4][16][20];          // per-wave 16x16 scratch
  float g[C], bb[C], rk[C], rq[C], sc[C];
};

__device__ __forceinline__ bf16x8 ld8p(const uint4* t, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(t) + row * (PQ * 16) + col * 2);
}

__global__ void __launch_bounds__(NT, 2)
gdn_prep_mfma(GdnParams p) {
  __shared__ __attribute__((aligned(16))) PrepSmem sm;
  float (*A)[AP] = reinterpret_cast<float (*)[AP]>(sm.QA);
  float (*T)[AP] = reinterpret_cast<float (*)[AP]>(sm.TT);
  bf16 (*aqk)[72] = reinterpret_cast<bf16 (*)[72]>(sm.TT);
  bf16 (*t1)[TP] = reinterpret_cast<bf16 (*)[TP]>(sm.TT);
  bf16 (*t2)[TP] = reinterpret_cast<bf16 (*)[TP]>(reinterpret_cast<unsigned char*>(sm.TT) + C * TP * 2);

  // last chunk first: when the state pass starts, the records it reads first
  // are the most recently written ones (still in the last-level cache)
  const int chunk = p.n_chunks - 1 - int(blockIdx.x), h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long t0 = (long long)chunk * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const size_t HD = size_t(p.H) * D;
  const unsigned tok_bytes = unsigned(HD * sizeof(bf16));
  const size_t tbase = ((size_t(b) * p.L + t0) * HD + size_t(h) * D) * sizeof(bf16);
  const size_t gbase = (size_t(b) * p.L + t0) * p.H + h;
  unsigned char* rec = p.ws + (size_t(b * p.H + h) * p.n_chunks + chunk) * p.rec_bytes;

  // ---- K, Q, V: direct loads into padded tiles (rows past the end repeat the last token) ----
  {
    const unsigned char* kb = static_cast<const unsigned char*>(p.k) + tbase;
    const unsigned char* qb = static_cast<const unsigned char*>(p.q) + tbase;
    const unsigned char* vb = static_cast<const unsigned char*>(p.v) + tbase;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int j = wave + 4 * i;
      if (j < PQ) {
        const unsigned off = tok_offset(slot_offset(64 * j + lane, PQ, 16, 256, C - 1), n - 1, tok_bytes);
        dma16(kb + off, &sm.K[64 * j]);
        dma16(qb + off, &sm.QA[64 * j]);
        dma16(vb + off, &sm.V[64 * j]);
      }
    }
  }
  if (wave == 0) {
    // gates: inclusive scan of log a over the chunk (one token per lane)
    float la = 0.f, bi = 0.f;
    if (lane < n) load_gates(p.a, p.b, gbase + size_t(lane) * p.H, p.gate_logits, kLogAFloor, la, bi);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (lane >= off) la += y;
    }
    sm.g[lane] = la;
    sm.bb[lane] = bi;
  }
  wait_vmem();
  __syncthreads();
  {
    // inverse norms: 4 threads per row, 32 elements each (four 16-byte reads per tile)
    const int row = tid >> 2, part = tid & 3;
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 kv = ld8p(sm.K, row, 32 * part + 8 * c);
      const bf16x8 qv = ld8p(sm.QA, row, 32 * part + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(kv[e]), y = static_cast<float>(qv[e]);
        sk += x * x;
        sq += y * y;
      }
    }
    sk += __shfl_xor(sk, 1, 4);
    sk += __shfl_xor(sk, 2, 4);
    sq += __shfl_xor(sq, 1, 4);
    sq += __shfl_xor(sq, 2, 4);
    if (part == 0) {
      sm.rk[row] = p.l2norm ? 1.f / sqrtf(sk + kL2Eps) : 1.f;
      sm.rq[row] = p.l2norm ? 1.f / sqrtf(sq + kL2Eps) : 1.f;
    }
  }
  __syncthreads();
  if (tid < C) sm.sc[tid] = sm.bb[tid] * __expf(sm.g[tid]) * sm.rk[tid];

  // ---- Gram products on raw bf16: wave w owns token rows 16w..16w+15 ----
  {
    bf16x8 ak[4], aq[4], bk[4][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      ak[ks] = ld8p(sm.K, 16 * wave + l16, 32 * ks + 8 * g);
      aq[ks] = ld8p(sm.QA, 16 * wave + l16, 32 * ks + 8 * g);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) bk[jb][ks] = ld8p(sm.K, 16 * jb + l16, 32 * ks + 8 * g);
    }
    f32x4 kk[4], qk[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      kk[jb] = qk[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kk[jb] = mfma16(ak[ks], bk[jb][ks], kk[jb]);
        qk[jb] = mfma16(aq[ks], bk[jb][ks], qk[jb]);
      }
    }
    float gi[4], ri[4], qi[4], bi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * wave + 4 * g + e;
      gi[e] = sm.g[i];
      ri[e] = sm.rk[i];
      qi[e] = sm.rq[i];
      bi[e] = sm.bb[i];
    }
    __syncthreads();   // every wave is done with the Q tile: it becomes A
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int j = 16 * jb + l16;
      const float gj = sm.g[j], rj = sm.rk[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * wave + 4 * g + e;
        const float ratio = j <= i ? __expf(gi[e] - gj) : 0.f;
        A[i][j] = j < i ? bi[e] * ratio * ri[e] * rj * kk[jb][e] : 0.f;
        aqk[i][j] = static_cast<bf16>(ratio * qi[e] * rj * qk[jb][e]);
      }
    }
  }
  __syncthreads();
  {
    // Aqk to the record (64 rows x 8 chunks of 16 B)
    bf16* dst = reinterpret_cast<bf16*>(rec + R::AQK);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + NT * i, row = e >> 3, c = e & 7;
      *reinterpret_cast<uint4*>(dst + row * C + c * 8) = *reinterpret_cast<const uint4*>(&aqk[row][c * 8]);
    }
  }
  __syncthreads();   // the staging is dead: the region becomes T

  // ---- T = (I + A)^-1, diagonal 16x16 blocks: wave w, lane c < 16 computes column c ----
  if (lane < 16) {
    const int o = 16 * wave, c = lane;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float4 row[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) row[q] = *reinterpret_cast<const float4*>(&A[o + r][o + 4 * q]);
      const float* a = reinterpret_cast<const float*>(row);
      float s = r == c ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < r; ++k) s -= a[k] * t[k];
      t[r] = r > c ? s : (r == c ? 1.f : 0.f);
      T[o + r][o + c] = t[r];
    }
  }
  __syncthreads();
  // off-diagonal blocks, level by level: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  for (int level = 1; level < 4; ++level) {
    const int i = wave, j = wave - level;
    if (j >= 0) {
      const int r = lane >> 2, cc = (lane & 3) * 4;
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k) {
        float4 arow[4], tr[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) arow[q] = *reinterpret_cast<const float4*>(&A[16 * i + r][16 * k + 4 * q]);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) tr[kk] = *reinterpret_cast<const float4*>(&T[16 * k + kk][16 * j + cc]);
        const float* a = reinterpret_cast<const float*>(arow);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          x[0] += a[kk] * tr[kk].x;
          x[1] += a[kk] * tr[kk].y;
          x[2] += a[kk] * tr[kk].z;
          x[3] += a[kk] * tr[kk].w;
        }
      }
      *reinterpret_cast<float4*>(&sm.X[wave][r][cc]) = make_float4(x[0], x[1], x[2], x[3]);
      // X is private to this wave and LDS executes a wave's accesses in order:
      // only the compiler must not move the reads above the writes
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float4 trow[4], xr[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) trow[q] = *reinterpret_cast<const float4*>(&T[16 * i + r][16 * i + 4 * q]);
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) xr[kk] = *reinterpret_cast<const float4*>(&sm.X[wave][kk][cc]);
      const float* tt = reinterpret_cast<const float*>(trow);
      float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) {
        y[0] += tt[kk] * xr[kk].x;
        y[1] += tt[kk] * xr[kk].y;
        y[2] += tt[kk] * xr[kk].z;
        y[3] += tt[kk] * xr[kk].w;
      }
      *reinterpret_cast<float4*>(&T[16 * i + r][16 * j + cc]) = make_float4(-y[0], -y[1], -y[2], -y[3]);
    }
    __syncthreads();
  }

  // ---- T' = T diag(b gamma / ||k||) and T'' = T diag(b) in bf16 (lower triangle) ----
  {
    const int i = tid >> 2, c0 = 16 * (tid & 3);
    float v1[16], v2[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 tq = *reinterpret_cast<const float4*>(&T[i][c0 + 4 * q]);
      const float4 sq4 = *reinterpret_cast<const float4*>(&sm.sc[c0 + 4 * q]);
      const float4 bq4 = *reinterpret_cast<const float4*>(&sm.bb[c0 + 4 * q]);
      const float tv[4] = {tq.x, tq.y, tq.z, tq.w}, sv[4] = {sq4.x, sq4.y, sq4.z, sq4.w},
                  bv[4] = {bq4.x, bq4.y, bq4.z, bq4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool lower = c0 + 4 * q + e <= i;
        v1[4 * q + e] = lower ? tv[e] * sv[e] : 0.f;
        v2[4 * q + e] = lower ? tv[e] * bv[e] : 0.f;
      }
    }
    __syncthreads();   // T is read: the region becomes T', T''
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bf16x4 w1 = {static_cast<bf16>(v1[4 * q]), static_cast<bf16>(v1[4 * q + 1]),
                         static_cast<bf16>(v1[4 * q + 2]), static_cast<bf16>(v1[4 * q + 3])};
      const bf16x4 w2 = {static_cast<bf16>(v2[4 * q]), static_cast<bf16>(v2[4 * q + 1]),
                         static_cast<bf16>(v2[4 * q + 2]), static_cast<bf16>(v2[4 * q + 3])};
      *reinterpret_cast<bf16x4*>(&t1[i][c0 + 4 * q]) = w1;
      *reinterpret_cast<bf16x4*>(&t2[i][c0 + 4 * q]) = w2;
    }
  }
  __syncthreads();

  // ---- W^T = K^T T'^T: wave w -> d_k blocks 2w, 2w+1 (A = K^T read transposed) ----
  {
    bf16* wn = reinterpret_cast<bf16*>(rec + R::WN);
    bf16x8 ka[2][2], tb8[2][4];
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const int jr = 32 * js + 8 * g;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int col = 16 * (2 * wave + mi) + 4 * (l16 & 3);
        ka[mi][js] = join(ld4p_tr<PQ>(sm.K, jr + (l16 >> 2), col), ld4p_tr<PQ>(sm.K, jr + 4 + (l16 >> 2), col));
      }
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const bf16* r = &t1[16 * ib + l16][jr];
        tb8[js][ib] = join(*reinterpret_cast<const bf16x4*>(r), *reinterpret_cast<const bf16x4*>(r + 4));
      }
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int mb = 2 * wave + mi;
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int js = 0; js < 2; ++js) acc = mfma16(ka[mi][js], tb8[js][ib], acc);
        // C layout: col = token i = 16ib + l16, rows d_k = 16mb + 4g + e -> Wn[i][d_k..d_k+3] = -W
        const int i = 16 * ib + l16;
        const bf16x4 v = {static_cast<bf16>(-acc[0]), static_cast<bf16>(-acc[1]), static_cast<bf16>(-acc[2]),
                          static_cast<bf16>(-acc[3])};
        *reinterpret_cast<bf16x4*>(wn + i * D + 16 * mb + 4 * g) = v;
      }
    }
  }
  // ---- U' = T'' V: wave w -> token rows 16w..16w+15, all 8 d_v blocks (B = V read transposed) ----
  {
    bf16* upt = reinterpret_cast<bf16*>(rec + R::UPT);
    bf16x8 ta[2];
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const bf16* r = &t2[16 * wave + l16][32 * js + 8 * g];
      ta[js] = join(*reinterpret_cast<const bf16x4*>(r), *reinterpret_cast<const bf16x4*>(r + 4));
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        const int jr = 32 * js + 8 * g, col = 16 * nb + 4 * (l16 & 3);
        const bf16x8 vb = join(ld4p_tr<PQ>(sm.V, jr + (l16 >> 2), col), ld4p_tr<PQ>(sm.V, jr + 4 + (l16 >> 2), col));
        acc = mfma16(ta[js], vb, acc);
      }
      // C layout: col = d_v = 16nb + l16, rows = tokens 16w + 4g + e -> UpT[d_v][tok..tok+3]
      const bf16x4 v = {static_cast<bf16>(acc[0]), static_cast<bf16>(acc[1]), static_cast<bf16>(acc[2]),
                        static_cast<bf16>(acc[3])};
      *reinterpret_cast<bf16x4*>(upt + (16 * nb + l16) * C + 16 * wave + 4 * g) = v;
    }
  }
  // ---- per-token scalars ----
  if (tid < C) {
    const int i = tid;
    const float gl = sm.g[C - 1];
    float* sqp = reinterpret_cast<float*>(rec + R::SQ);
    float* skp = reinterpret_cast<float*>(rec + R::SK);
    sqp[i] = i < n ? __expf(sm.g[i]) * sm.rq[i] : 0.f;
    skp[i] = i < n ? __expf(gl - sm.g[i]) * sm.rk[i] : 0.f;
    if (i == 0) *reinterpret_cast<float*>(rec + R::GC) = __expf(gl);
  }
}

// ---------------------------------------------------------------------------
// kernel 2: the chunk-to-chunk state pass
// ---------------------------------------------------------------------------

// One chunk's operands in LDS, rows padded so that 16 lanes reading one
// column of 16 rows hit distinct banks: 272-byte rows for -W and q, 288-byte
// rows for k (read transposed), 144-byte rows for the 64-wide tiles. Tiles
// arrive by direct global -> LDS loads: a wave instruction writes 1 KB
// contiguously (lane i at byte 16 i), so padded tiles are filled as runs of
// 64 chunk slots, each lane loading the chunk its slot holds (pad slots load
// a harmless in-row chunk).
constexpr int PW = 17;   // chunk slots per row: -W and q
constexpr int PK = 18;   // k
constexpr int PS = 9;    // Aqk, U'^T rows
constexpr int NV = 16;   // value channels per workgroup (one wave)
constexpr int kChainXcds = 8;
struct ChainBuf {
  uint4 Wn[C * PW];
  uint4 Q[C * PW];
  uint4 K[C * PK];
  uint4 Aqk[C * PS];
  uint4 UpT[NV * PS];
  float sc[2 * C + 32];  // sq[C], sk[C], gC
};
struct ChainSmem {
  ChainBuf buf[2];
  bf16x8 stage[2][4][64];    // bf16 S^T published by the state wave, per lane, by chunk parity
  unsigned pf_scratch[64];   // target of the L2 prefetch loads (never read)
};

// Lane offsets of the direct loads of one chunk (the same for every chunk).
// Record tiles use (row * 256 + chunk * 16) form; q and k rows are tokens of
// the input tensors, so their offsets are rescaled to the token stride. Full
// chunks use the precomputed 32-bit offsets on a scalar base (no per-load
// vector arithmetic); the ragged last chunk clamps rows to its last token.
struct DmaPlan {
  unsigned w[PW], k[PK], aqk[PS], upt[3];
  unsigned qo[PW], ko[PK];
};

__device__ __forceinline__ void make_plan(DmaPlan& pl, int lane, unsigned tok_bytes) {
#pragma unroll
  for (int j = 0; j < PW; ++j) {
    pl.w[j] = slot_offset(64 * j + lane, PW, 16, 256, C - 1);
    pl.qo[j] = tok_offset(pl.w[j], C - 1, tok_bytes);
  }
#pragma unroll
  for (int j = 0; j < PK; ++j) {
    pl.k[j] = slot_offset(64 * j + lane, PK, 16, 256, C - 1);
    pl.ko[j] = tok_offset(pl.k[j], C - 1, tok_bytes);
  }
#pragma unroll
  for (int j = 0; j < PS; ++j) pl.aqk[j] = slot_offset(64 * j + lane, PS, 8, 128, C - 1);
#pragma unroll
  for (int j = 0; j < 3; ++j) pl.upt[j] = slot_offset(64 * j + lane, PS, 8, 128, NV - 1);
}

// Buffer resource over [base, base + bytes): loads through it take a 32-bit
// lane offset plus a scalar offset (no per-lane 64-bit address arithmetic),
// and lanes past the end read zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const unsigned n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : unsigned(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(n), 0x00020000);
}
__device__ __forceinline__ void dma16r(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_base), 16, voff, soff, 0,
                                           0);
}

// One chunk's operands into buf: the record's -W, Aqk, U' slice and scales,
// and the q, k rows of its tokens (qk_bytes: bytes of q and k from the
// chunk's first token to the end of the tensors).
__device__ __forceinline__ void issue_chunk(ChainBuf& buf, const DmaPlan& pl, const unsigned char* rec,
                                            size_t rec_bytes, const unsigned char* qb, const unsigned char* kb,
                                            size_t qk_bytes, int vblk, int lane, int n, unsigned tok_bytes) {
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, rec_bytes);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, qk_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, qk_bytes);
#pragma unroll
  for (int j = 0; j < PW; ++j) dma16r(rr, pl.w[j], unsigned(R::WN), &buf.Wn[64 * j]);
  if (n == C) {
#pragma unroll
    for (int j = 0; j < PW; ++j) dma16r(rq, pl.qo[j], 0u, &buf.Q[64 * j]);
#pragma unroll
    for (int j = 0; j < PK; ++j) dma16r(rk, pl.ko[j], 0u, &buf.K[64 * j]);
  } else {
#pragma unroll
    for (int j = 0; j < PW; ++j) dma16r(rq, tok_offset(pl.w[j], n - 1, tok_bytes), 0u, &buf.Q[64 * j]);
#pragma unroll
    for (int j = 0; j < PK; ++j) dma16r(rk, tok_offset(pl.k[j], n - 1, tok_bytes), 0u, &buf.K[64 * j]);
  }
#pragma unroll
  for (int j = 0; j < PS; ++j) dma16r(rr, pl.aqk[j], unsigned(R::AQK), &buf.Aqk[64 * j]);
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (64 * j + lane < NV * PS) dma16r(rr, pl.upt[j], unsigned(R::UPT + size_t(NV * vblk) * 128), &buf.UpT[64 * j]);
  if (lane < 33) dma16r(rr, 16u * unsigned(lane), unsigned(R::SQ), &buf.sc[0]);
}

// Workgroup barrier for LDS accesses made by the waves' own instructions:
// they complete (lgkmcnt(0)) before it, and the compiler moves no memory
// access across it. Direct loads into LDS are waited for explicitly by the
// loader (a release fence here would also make the prefetch wave wait for its
// L2 prefetches every chunk), and global stores in flight are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// L2 prefetch of one chunk's operands: the record (325 lines of 128 B up to
// gamma_C) and the q and k rows of its tokens (2 lines each). The 8
// workgroups of a head split the lines (part = value block); each lane
// touches one line with a 4-byte direct load into a scratch LDS word.
constexpr int kRecLines = int((R::GC + 4 + 127) / 128);
constexpr int kPrefetchLines = kRecLines + 4 * C;
static_assert(kPrefetchLines <= 2 * 64 * (D / NV), "prefetch lanes");
__device__ __forceinline__ void prefetch_chunk(const unsigned char* rec, const unsigned char* qb,
                                               const unsigned char* kb, int part, int lane, int n,
                                               unsigned tok_bytes, unsigned* scratch) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = part * 128 + 64 * j + lane;
    const unsigned char* src = rec;
    if (idx < kRecLines) {
      src = rec + 128 * idx;
    } else if (idx < kPrefetchLines) {
      const int t = idx - kRecLines, which = t >> 7, tok = min((t & 127) >> 1, n - 1);
      src = (which ? kb : qb) + unsigned(tok) * tok_bytes + 128u * unsigned(t & 1);
    }
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                     (__attribute__((address_space(3))) void*)(scratch), 4, 0, 0);
  }
}

// Four waves per workgroup, one per SIMD:
//   wave 0 (state)   U = U' - W S^T and S <- gamma_C S + K^T diag(sk) U; it
//                    publishes the bf16 copy of each new S in LDS;
//   wave 1 (output)  recomputes U from that copy (same operands, same
//                    products, so the same U) and writes O = diag(sq) Q S^T + Aqk U;
//   wave 2 (loader)  loads chunk c + 1 into the other LDS buffer;
//   wave 3           prefetches chunk c + kPrefetchAhead into L2.
// One barrier per chunk hands the buffers and the published state over.
constexpr int kChainWaves = 4;
constexpr int kPrefetchAhead = 4;

// -W tile (A operand of W S^T) and the U' slice (its initial value) of this lane.
__device__ __forceinline__ void load_u_operands(const ChainBuf& B, int g, int l16, bf16x8 (&aw)[4][4],
                                                bf16x4 (&upv)[4]) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int row = 16 * tb + l16;
    upv[tb] = ld4p<PS>(B.UpT, l16, 16 * tb + 4 * g);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      aw[tb][ks] = join(ld4p<PW>(B.Wn, row, 32 * ks + 4 * g), ld4p<PW>(B.Wn, row, 32 * ks + 16 + 4 * g));
  }
}

// U = U' - W S^T in C layout: u[tb] holds tokens 16tb + 4g + e of channel v0 + l16.
__device__ __forceinline__ void compute_u(const bf16x8 (&aw)[4][4], const bf16x4 (&upv)[4], const bf16x8 (&sb)[4],
                                          f32x4 (&u)[4]) {
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    u[tb] = f32x4{static_cast<float>(upv[tb][0]), static_cast<float>(upv[tb][1]), static_cast<float>(upv[tb][2]),
                  static_cast<float>(upv[tb][3])};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) u[tb] = mfma16(aw[tb][ks], sb[ks], u[tb]);
  }
}

// bf16 copy of S^T: K-step ks takes blocks 2ks, 2ks+1 (d_k = 32ks + 16(i/4) + 4g + i%4).
// The 16x16x32 A and B layouts coincide, so it is the B operand of W S^T
// (S^T, columns d_v) and the A operand of S q^T (S, rows d_v) alike.
__device__ __forceinline__ void state_bf16(const f32x4 (&st)[8], bf16x8 (&sb)[4]) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sb[ks][e] = static_cast<bf16>(st[2 * ks][e]);
      sb[ks][4 + e] = static_cast<bf16>(st[2 * ks + 1][e]);
    }
}

template <typename Tout>
__global__ void __launch_bounds__(64 * kChainWaves, 1)
gdn_chain_mfma(GdnParams p) {
  __shared__ __attribute__((aligned(16))) ChainSmem sm;
  // XCD-aware: the 8 workgroups of a head get blockIdx with the same value mod 8
  const int xcd = blockIdx.x % kChainXcds, slot = blockIdx.x / kChainXcds;
  const int vblk = slot % (D / NV);
  const int bh = (slot / (D / NV)) * kChainXcds + xcd;
  if (bh >= p.B * p.H) return;
  const int b = bh / p.H, h = bh % p.H;
  if (skipped(p.skip, b)) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int v0 = NV * vblk;   // this workgroup's value channels v0 .. v0+15
  const size_t HD = size_t(p.H) * D;
  const size_t sbase = (size_t(b) * p.H + h) * D * D;
  const unsigned tok_bytes = unsigned(HD * sizeof(bf16));
  auto rec_of = [&](int chunk) {
    return p.ws + (size_t(b * p.H + h) * p.n_chunks + chunk) * p.rec_bytes;
  };
  auto tok_base = [&](int chunk) {
    return ((size_t(b) * p.L + (long long)chunk * C) * HD + size_t(h) * D) * sizeof(bf16);
  };
  auto chunk_len = [&](int chunk) {
    const long long t0 = (long long)chunk * C;
    return int(p.L - t0 < C ? p.L - t0 : C);
  };

  if (wave == 2) {
    // loader: chunk c + 1 into buf[(c + 1) & 1] while chunk c is computed
    DmaPlan plan;
    make_plan(plan, lane, tok_bytes);
    const size_t qk_total = size_t(p.B) * size_t(p.L) * HD * sizeof(bf16);
    auto issue = [&](int chunk) {
      const size_t tb = tok_base(chunk);
      issue_chunk(sm.buf[chunk & 1], plan, rec_of(chunk), p.rec_bytes, static_cast<const unsigned char*>(p.q) + tb,
                  static_cast<const unsigned char*>(p.k) + tb, qk_total - tb, vblk, lane, chunk_len(chunk),
                  tok_bytes);
    };
    issue(0);
    wait_vmem();
    lds_barrier();
    for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
      if (chunk + 1 < p.n_chunks) issue(chunk + 1);
      wait_vmem();
      lds_barrier();
    }
    return;
  }
  if (wave == 3) {
    // L2 prefetcher: never waits for its loads inside the loop
    auto pf = [&](int chunk) {
      const size_t tb = tok_base(chunk);
      prefetch_chunk(rec_of(chunk), static_cast<const unsigned char*>(p.q) + tb,
                     static_cast<const unsigned char*>(p.k) + tb, vblk, lane, chunk_len(chunk), tok_bytes,
                     sm.pf_scratch);
    };
    for (int c = 1; c < kPrefetchAhead && c < p.n_chunks; ++c) pf(c);
    lds_barrier();
    for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
      if (chunk + kPrefetchAhead < p.n_chunks) pf(chunk + kPrefetchAhead);
      lds_barrier();
    }
    wait_vmem();
    return;
  }

  if (wave == 0) {
    // state wave: S^T slice in C layout, block mb holds d_k rows 16mb + 4g + e, column d_v = v0 + l16
    f32x4 st[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      if (p.S0) {
        const float4 v = *reinterpret_cast<const float4*>(p.S0 + sbase + size_t(v0 + l16) * D + 16 * mb + 4 * g);
        st[mb] = f32x4{v.x, v.y, v.z, v.w};
      } else {
        st[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    bf16x8 sb[4];
    state_bf16(st, sb);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sm.stage[0][ks][lane] = sb[ks];
    lds_barrier();   // chunk 0 has landed; the initial state is published
    for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
      const ChainBuf& B = sm.buf[chunk & 1];
      bf16x8 aw[4][4];
      bf16x4 upv[4];
      load_u_operands(B, g, l16, aw, upv);
      f32x4 skv[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) skv[tb] = *reinterpret_cast<const f32x4*>(&B.sc[C + 16 * tb + 4 * g]);
      const float gc = B.sc[2 * C];
      __builtin_amdgcn_sched_barrier(0);
      f32x4 u[4];
      compute_u(aw, upv, sb, u);
      // k^T (A operand of the state update), read while the U products run
      bf16x8 ak[8][2];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          const int col = 16 * mb + 4 * (l16 & 3);
          ak[mb][js] = join(ld4p_tr<PK>(B.K, 32 * js + 4 * g + (l16 >> 2), col),
                            ld4p_tr<PK>(B.K, 32 * js + 16 + 4 * g + (l16 >> 2), col));
        }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 usb[2];
#pragma unroll
      for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          usb[js][e] = static_cast<bf16>(u[2 * js][e] * skv[2 * js][e]);
          usb[js][4 + e] = static_cast<bf16>(u[2 * js + 1][e] * skv[2 * js + 1][e]);
        }
      // S^T <- gamma_C S^T + K^T diag(sk) U
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st[mb][e] *= gc;
#pragma unroll
        for (int js = 0; js < 2; ++js) st[mb] = mfma16(ak[mb][js], usb[js], st[mb]);
      }
      state_bf16(st, sb);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sm.stage[(chunk + 1) & 1][ks][lane] = sb[ks];
      lds_barrier();   // buf[chunk & 1] is free; chunk + 1 has landed; S of chunk + 1 is published
    }
    if (p.S_out) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        *reinterpret_cast<float4*>(p.S_out + sbase + size_t(v0 + l16) * D + 16 * mb + 4 * g) =
            make_float4(st[mb][0], st[mb][1], st[mb][2], st[mb][3]);
    }
    return;
  }

  // output wave
  Tout* o = static_cast<Tout*>(p.o);
  lds_barrier();
  for (int chunk = 0; chunk < p.n_chunks; ++chunk) {
    const ChainBuf& B = sm.buf[chunk & 1];
    const long long t0 = (long long)chunk * C;
    const int n = chunk_len(chunk);
    bf16x8 sb[4], aw[4][4];
    bf16x4 upv[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) sb[ks] = sm.stage[chunk & 1][ks][lane];
    load_u_operands(B, g, l16, aw, upv);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 u[4];
    compute_u(aw, upv, sb, u);
    // q and Aqk rows (B operands of S q^T and U^T Aqk^T) and the query scales
    bf16x8 aq[4][4], aa[4][2];
    float sqs[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int row = 16 * tb + l16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        aq[tb][ks] = join(ld4p<PW>(B.Q, row, 32 * ks + 4 * g), ld4p<PW>(B.Q, row, 32 * ks + 16 + 4 * g));
#pragma unroll
      for (int js = 0; js < 2; ++js)
        aa[tb][js] = join(ld4p<PS>(B.Aqk, row, 32 * js + 4 * g), ld4p<PS>(B.Aqk, row, 32 * js + 16 + 4 * g));
      sqs[tb] = B.sc[row];
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 ub[2];
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ub[js][e] = static_cast<bf16>(u[2 * js][e]);
        ub[js][4 + e] = static_cast<bf16>(u[2 * js + 1][e]);
      }
    // O^T = (S q^T) diag(sq) + U^T Aqk^T: lane holds channels v0 + 4g + e of token 16tb + l16
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) x = mfma16(sb[ks], aq[tb][ks], x);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= sqs[tb];
#pragma unroll
      for (int js = 0; js < 2; ++js) x = mfma16(ub[js], aa[tb][js], x);
      const int tok = 16 * tb + l16;
      if (tok < n) {
        Tout* dst = o + (size_t(b) * p.L + t0 + tok) * HD + size_t(h) * D + v0 + 4 * g;
        if constexpr (sizeof(Tout) == 2) {
          *reinterpret_cast<bf16x4*>(dst) = bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]),
                                                   static_cast<bf16>(x[2]), static_cast<bf16>(x[3])};
        } else {
          *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
        }
      }
    }
    lds_barrier();
  }
}

}  // namespace

hipError_t launch_gdn_mfma(const GdnParams& p, int out_dt, hipStream_t st) {
  if (p.rec_bytes < R::BYTES) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn_prep_mfma, dim3(p.n_chunks, p.H, p.B), dim3(NT), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int heads_per_xcd = (p.B * p.H + kChainXcds - 1) / kChainXcds;
  const dim3 grid(unsigned(kChainXcds * heads_per_xcd * (D / NV)));
  if (out_dt == HLTA_BF16)
    hipLaunchKernelGGL((gdn_chain_mfma<bf16>), grid, dim3(64 * kChainWaves), 0, st, p);
  else
    hipLaunchKernelGGL((gdn_chain_mfma<float>), grid, dim3(64 * kChainWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace hlta
