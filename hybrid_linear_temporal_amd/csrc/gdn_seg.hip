// Gated delta rule with bf16 MFMA on gfx950 (bf16 inputs, d = 128, chunk 64),
// parallel over the sequence as well as over heads.
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
// The state update is affine in S: S <- S M_c + N_c with
// M_c = gamma_C I - W^T diag(gamma_C / gamma) K^. A run of chunks therefore
// composes to one affine map S_end = S_start M + N, which lets the chunk chain
// of one head run in segments side by side. Four launches:
//
//   gdn_tinv_kernel: every chunk independently (no state): the triangular
//     inverse T scaled as T'' = T diag(b) and T' = T diag(b gamma / ||k||),
//     with the chunk's gate prefix sums, b and inverse key norms, written as
//     a 13,056-byte record in the exact MFMA operand order the later passes
//     read (so no pass repeats the inverse, the part of a chunk with the
//     longest dependent chains);
//   gdn_seg_kernel<false> (pass 1): every segment but the last, one
//     workgroup running two chains over the same tiles: from S = 0 (its end
//     state is N) and from S = I with the value term dropped (its end state
//     is M);
//   gdn_seg_scan (pass 2): per head and 16 state rows, S_{g+1} = S_g M_g + N_g
//     over the segments in order (fp32 accuracy from split bf16 products);
//   gdn_seg_kernel<true> (pass 3): every segment from its true start state,
//     writing o_gdn (and S_out from the last segment).
//
// In passes 1 and 3 a workgroup owns the whole 128 x 128 state of its segment
// (pass 1: both states; wave w: 32 columns of S^T in MFMA accumulator layout,
// fp32 in registers), so a chunk's q, k, v
// are loaded once and W, U' and the causal q.k matrix are formed on chip from
// the record; nothing per chunk but the record goes through memory.
#include <type_traits>

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

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 join(const bf16x4& lo, const bf16x4& hi) {
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& x) {
  return bf16x4{static_cast<bf16>(x[0]), static_cast<bf16>(x[1]), static_cast<bf16>(x[2]),
                static_cast<bf16>(x[3])};
}

// Transposed LDS read (gfx950): inside each group of 16 lanes, lane j gets
// element j%4 of the 4-element rows addressed by lanes 4e + j/4, e = 0..3.
__device__ __forceinline__ bf16x4 ld_tr(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ void dma16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)

// Workgroup barrier for LDS traffic (direct loads are waited for separately).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Token tiles (64 rows of 128 bf16) in LDS have 272-byte rows: 16 data slots
// of 16 bytes and a pad slot, so 16 lanes reading one column of 16 rows hit
// distinct banks.
constexpr int PQ = 17;                       // 16-byte slots per tile row
constexpr int TILE = C * PQ;                 // uint4 per tile
constexpr int AP = 68;                       // fp32 pitch of A / T
constexpr int QP = 72;                       // bf16 pitch of Aqk
static_assert(C * AP * 4 == TILE * 16, "A/T fill one tile region");

__device__ __forceinline__ bf16x4 ld4(const uint4* t, int row, int col) {
  return *reinterpret_cast<const bf16x4*>(reinterpret_cast<const char*>(t) + row * (PQ * 16) + col * 2);
}
__device__ __forceinline__ bf16x4 ld4_tr(const uint4* t, int row, int col) {
  return ld_tr(reinterpret_cast<const char*>(t) + row * (PQ * 16) + col * 2);
}
__device__ __forceinline__ bf16x8 ld8(const uint4* t, int row, int col) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(t) + row * (PQ * 16) + col * 2);
}
__device__ __forceinline__ void st4(uint4* t, int row, int col, const bf16x4& v) {
  *reinterpret_cast<bf16x4*>(reinterpret_cast<char*>(t) + row * (PQ * 16) + col * 2) = v;
}

// Source byte offset of tile slot P (row P / PQ, 16-byte column P % PQ; the
// pad slot loads a harmless in-row chunk), rows past the chunk's last token
// repeating that token.
__device__ __forceinline__ unsigned slot_src(int P, int last_row, unsigned tok_bytes) {
  int row = P / PQ, ch = P - row * PQ;
  if (ch > 15) ch = 15;
  if (row > last_row) row = last_row;
  return unsigned(row) * tok_bytes + unsigned(ch) * 16u;
}

// Direct loads of one token tile (rows t0 .. t0+63 of one head) into LDS,
// wave w issuing slots 64(w + 4i) .. +63.
__device__ __forceinline__ void load_tile(const unsigned char* src, uint4* tile, int wave, int lane, int n,
                                          unsigned tok_bytes) {
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int j = wave + 4 * i;
    if (j < PQ) dma16(src + slot_src(64 * j + lane, n - 1, tok_bytes), &tile[64 * j]);
  }
}

// ---------------------------------------------------------------------------
// per-chunk records
// ---------------------------------------------------------------------------
// A record holds what every later pass needs of a chunk and that does not
// depend on the state: T'' = T diag(b) and T' = T diag(b gamma / ||k||), the
// B operands of U'^T = V^T T''^T and W^T = K^T T'^T, then the chunk's gate
// prefix sums g, its b and its inverse key norms (fp32, 64 each). Tile (js,
// ib) of an operand (tokens j in 32js .. 32js+31 of the reduction, tokens i in
// 16ib .. 16ib+15 of the output) gives lane (g, l16) the 8 values
// T[16ib + l16][32js + 8g .. +7]; the matrices are lower triangular, so only
// the six tiles with 32js <= 16ib + 15 exist, stored 64 lanes x 16 bytes each
// in the order (0,0) (0,1) (0,2) (1,2) (0,3) (1,3).
constexpr int kRecTiles = 6;
constexpr int kRecTileBytes = kRecTiles * 64 * 16;
constexpr int kRecTpp = 0;                                // T''
constexpr int kRecTp = kRecTileBytes;                     // T'
constexpr int kRecG = 2 * kRecTileBytes;                  // g[64]
constexpr int kRecB = kRecG + 256;                        // b[64]
constexpr int kRecRk = kRecB + 256;                       // 1/||k||, [64]
constexpr int kRecBytes = kRecRk + 256;
static_assert(kRecBytes % 256 == 0, "records stay 256-byte aligned");
__device__ __forceinline__ int rec_tile(int js, int ib) { return ib < 2 ? ib : 2 * ib - 2 + js; }

// ---------------------------------------------------------------------------
// kernel T: per chunk, T = (I + A)^-1 and its record
// ---------------------------------------------------------------------------
// LDS 23.5 KB, so six workgroups share a CU and the long dependent chains of
// the inverse of one chunk overlap with the others'. Kt holds the chunk's k
// rows until the Gram products have read them; the same bytes (R1) then hold
// A in its strictly lower 16x16 blocks (fp32) and T transposed in the rest:
// element (m, n) with n at or right of m's diagonal block is T[n][m]. XA first
// holds the diagonal blocks of A transposed (for the column-oriented solve),
// then per-wave 16x16 scratch.
struct TinvSmem {
  union {
    uint4 Kt[TILE];
    uint4 R1[TILE];
  };
  float XA[4 * 16 * 20];
  float g[C], bb[C], rk[C], sc[C];
};
static_assert(sizeof(TinvSmem) <= 160 * 1024 / 6, "six workgroups per CU");

// x = hi + lo with hi, lo in bf16 (about 16 significant bits together)
__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<bf16>(x[e]);
    lo[e] = static_cast<bf16>(x[e] - static_cast<float>(hi[e]));
  }
}

// c += a b with both factors split: hi*hi + hi*lo + lo*hi in fp32 accumulation
__device__ __forceinline__ f32x4 mfma_split(const float (&a)[8], const float (&b)[8], f32x4 c) {
  bf16x8 ah, al, bh, bl;
  split_bf16(a, ah, al);
  split_bf16(b, bh, bl);
  c = mfma16(ah, bh, c);
  c = mfma16(ah, bl, c);
  return mfma16(al, bh, c);
}

__global__ void __launch_bounds__(NT, 6)
gdn_tinv_kernel(GdnParams p, unsigned char* recs) {
  __shared__ __attribute__((aligned(16))) TinvSmem sm;
  const int chunk = int(blockIdx.x), h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long long t0 = (long long)chunk * C;
  const int n = int(p.L - t0 < C ? p.L - t0 : C);
  const size_t HD = size_t(p.H) * D;
  const unsigned tok_bytes = unsigned(HD * sizeof(bf16));
  const size_t tbase = ((size_t(b) * p.L + t0) * HD + size_t(h) * D) * sizeof(bf16);
  float (*R)[AP] = reinterpret_cast<float (*)[AP]>(sm.R1);
  float (*ADT)[16][16] = reinterpret_cast<float (*)[16][16]>(sm.XA);

  load_tile(static_cast<const unsigned char*>(p.k) + tbase, sm.Kt, wave, lane, n, tok_bytes);
  if (wave == 0) {
    float la = 0.f, bi = 0.f;
    if (lane < n)
      load_gates(p.a, p.b, (size_t(b) * p.L + t0 + lane) * p.H + h, p.gate_logits, kLogAFloor, la, bi);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(la, off);
      if (lane >= off) la += y;
    }
    sm.g[lane] = la;
    sm.bb[lane] = bi;
  }
  wait_vmem();
  lds_barrier();
  {
    // inverse key norms: 4 threads per row
    const int row = tid >> 2, part = tid & 3;
    float s2 = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bf16x8 kv = ld8(sm.Kt, row, 32 * part + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) s2 += static_cast<float>(kv[e]) * static_cast<float>(kv[e]);
    }
    s2 += __shfl_xor(s2, 1, 4);
    s2 += __shfl_xor(s2, 2, 4);
    if (part == 0) {
      const float rk = p.l2norm ? 1.f / sqrtf(s2 + kL2Eps) : 1.f;
      sm.rk[row] = rk;
      sm.sc[row] = sm.bb[row] * __expf(sm.g[row]) * rk;   // columns of T'
    }
  }
  lds_barrier();
  // ---- A from K K^T on raw bf16 (exact products, fp32 sums): wave w owns rows 16w ..;
  //      the four column blocks as independent chains, those right of the diagonal unused ----
  {
    bf16x8 ak[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ak[ks] = ld8(sm.Kt, 16 * wave + l16, 32 * ks + 8 * g);
    f32x4 kk[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) kk[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) kk[jb] = mfma16(ak[ks], ld8(sm.Kt, 16 * jb + l16, 32 * ks + 8 * g), kk[jb]);
    lds_barrier();   // every wave has read Kt, whose bytes R now takes over
    float gi[4], bri[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 16 * wave + 4 * g + e;
      gi[e] = sm.g[i];
      bri[e] = sm.bb[i] * sm.rk[i];
    }
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      if (jb > wave) continue;
      // C layout: row i = 16 wave + 4g + e, column j = 16 jb + l16
      const int j = 16 * jb + l16;
      const float gj = sm.g[j], rj = sm.rk[j];
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * wave + 4 * g + e;
        a[e] = j < i ? bri[e] * __expf(gi[e] - gj) * rj * kk[jb][e] : 0.f;
        if (jb < wave) R[i][j] = a[e];
      }
      // the diagonal block transposed: row k holds column k of A
      if (jb == wave) *reinterpret_cast<f32x4*>(&ADT[wave][l16][4 * g]) = a;
    }
  }
  lds_barrier();
  // ---- diagonal blocks: lane c < 16 of wave w solves column c of T_ww ----
  if (lane < 16) {
    // forward substitution by columns of A_ww: the updates of one step are
    // independent, so the dependent chain is 15 steps long; column k + 1 is
    // read while step k runs (the fences keep the compiler from hoisting all
    // fifteen reads at once)
    const int o16 = 16 * wave, c = lane;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = r == c ? 1.f : 0.f;
    f32x4 cur[4], nxt[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) cur[q4] = *reinterpret_cast<const f32x4*>(&ADT[wave][0][4 * q4]);
#pragma unroll
    for (int k = 0; k < 15; ++k) {
      if (k + 1 < 15) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) nxt[q4] = *reinterpret_cast<const f32x4*>(&ADT[wave][k + 1][4 * q4]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = k + 1; r < 16; ++r) t[r] -= cur[r >> 2][r & 3] * t[k];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
    }
    // T_ww transposed: row c of the block holds column c of T_ww
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(&R[o16 + c][o16 + 4 * q4]) =
          make_float4(t[4 * q4], t[4 * q4 + 1], t[4 * q4 + 2], t[4 * q4 + 3]);
  }
  lds_barrier();
  // ---- off-diagonal blocks level by level on split-bf16 MFMA:
  //      X = sum_{m in block rows j .. i-1} A[16i + r][m] T[m][16j + c],  T_ij = -T_ii X ----
  for (int level = 1; level < 4; ++level) {
    const int i = wave, j = wave - level;
    if (j >= 0) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int m0 = 16 * j; m0 < 16 * i; m0 += 32) {
        // A operand: row 16i + l16, columns m0 + 8g ..; B operand: T[m0 + 8g ..][16j + l16],
        // which is row 16j + l16 of the region (T transposed); past 16i both are 0
        float av[8], bv[8];
        const bool valid = m0 + 8 * g < 16 * i;
        if (valid) {
          const float4 a0 = *reinterpret_cast<const float4*>(&R[16 * i + l16][m0 + 8 * g]);
          const float4 a1 = *reinterpret_cast<const float4*>(&R[16 * i + l16][m0 + 8 * g + 4]);
          const float4 b0 = *reinterpret_cast<const float4*>(&R[16 * j + l16][m0 + 8 * g]);
          const float4 b1 = *reinterpret_cast<const float4*>(&R[16 * j + l16][m0 + 8 * g + 4]);
          av[0] = a0.x; av[1] = a0.y; av[2] = a0.z; av[3] = a0.w; av[4] = a1.x; av[5] = a1.y; av[6] = a1.z; av[7] = a1.w;
          bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w; bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) av[e] = bv[e] = 0.f;
        }
        x = mfma_split(av, bv, x);
      }
      // Y^T = X^T T_ii^T: reduction slots 8g + q hold r = 4g + q for q < 4 (X in
      // accumulator layout is X^T's A operand that way), the others are 0
      float xa[8], tb[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xa[q] = x[q];
        xa[4 + q] = 0.f;
        tb[q] = R[16 * i + 4 * g + q][16 * i + l16];   // T_ii[l16][4g + q]
        tb[4 + q] = 0.f;
      }
      const f32x4 y = mfma_split(xa, tb, f32x4{0.f, 0.f, 0.f, 0.f});
      // lane holds Y[l16][4g + e]; T_ij = -Y goes (transposed) to R[16j + 4g + e][16i + l16]
#pragma unroll
      for (int e = 0; e < 4; ++e) R[16 * j + 4 * g + e][16 * i + l16] = -y[e];
    }
    lds_barrier();
  }
  // ---- the record (wave w writes tiles w and w + 4 of T'' and T'; wave 0 the scalars) ----
  unsigned char* rec = recs + (size_t(b * p.H + h) * p.n_chunks + chunk) * kRecBytes;
#pragma unroll
  for (int rep = 0; rep < 2; ++rep) {
    const int t = wave + 4 * rep;
    if (t < kRecTiles) {
      const int ib = t < 2 ? t : 2 + (t - 2) / 2, js = t < 2 ? 0 : (t - 2) % 2;
      const int j0 = 32 * js + 8 * g;
      bf16x8 v2, v1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // T[16ib + l16][j0 + e] = region (j0 + e, 16ib + l16); right of the diagonal T is 0
        const int jj = j0 + e;
        const float tv = jj <= 16 * ib + l16 ? R[jj][16 * ib + l16] : 0.f;
        v2[e] = static_cast<bf16>(tv * sm.bb[jj]);
        v1[e] = static_cast<bf16>(tv * sm.sc[jj]);
      }
      *reinterpret_cast<bf16x8*>(rec + kRecTpp + (size_t(t) * 64 + lane) * 16) = v2;
      *reinterpret_cast<bf16x8*>(rec + kRecTp + (size_t(t) * 64 + lane) * 16) = v1;
    }
  }
  if (wave == 0) {
    reinterpret_cast<float*>(rec + kRecG)[lane] = sm.g[lane];
    reinterpret_cast<float*>(rec + kRecB)[lane] = sm.bb[lane];
    reinterpret_cast<float*>(rec + kRecRk)[lane] = sm.rk[lane];
  }
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

// ---------------------------------------------------------------------------
// passes 1 and 3
// ---------------------------------------------------------------------------
// LDS (about 80 KB in pass 3, two workgroups per CU), per chunk:
//   Kt   k rows (raw)
//   Qt   q rows (raw, pass 3 only)
//   Vt   v rows (raw), then U' (rows = tokens)
//   R1   the chunk's record, then -W (rows = tokens)
//   XA   Aqk (bf16, pass 3 only)
// and the per-token scales below. They are separate arrays, not members of
// one struct, so the compiler can tell a direct load into one of them from
// reads of the others: the next chunk's tiles are loaded while this chunk's
// last products still read the other tiles, with no wait for those loads.
struct __attribute__((aligned(16))) SegVec {
  float sq[C], sk[C], rq[C];
  float gC;
};

// State columns per wave: S^T is d_k (128 rows) x 128 columns, wave w owns
// columns 32w .. 32w+31 as 8 x 2 tiles of 16 x 16 in MFMA accumulator layout
// (tile (mb, nb): rows d_k 16mb + 4g + e, column 32w + 16nb + l16).
struct State {
  f32x4 st[8][2];
};

// bf16 copy of the state slice: K-step ks takes tiles 2ks, 2ks+1 (d_k =
// 32ks + 16(i/4) + 4g + i%4). The 16x16x32 A and B layouts coincide, so it is
// the B operand of W S^T (columns = the wave's state columns) and the A
// operand of S Q^T (rows = the same columns) alike; every operand it meets
// is read from LDS in that permuted d_k order.
__device__ __forceinline__ void state_bf16(const State& s, bf16x8 (&sb)[2][4]) {
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sb[nb][ks][e] = static_cast<bf16>(s.st[2 * ks][nb][e]);
        sb[nb][ks][4 + e] = static_cast<bf16>(s.st[2 * ks + 1][nb][e]);
      }
}

// Segment g's chunk range.
__device__ __forceinline__ void seg_range(int g, int seg_chunks, int n_chunks, int& c0, int& c1) {
  c0 = g * seg_chunks;
  c1 = c0 + seg_chunks < n_chunks ? c0 + seg_chunks : n_chunks;
}

// Map slots of the workspace, 2G - 1 d x d fp32 matrices per (b, h): for each
// segment g < G-1, slot 2g first holds N_g (row-major, rows = state rows),
// then S_{g+1} (written over it by the scan), and slot 2g+1 holds M_g
// transposed (row j, column r = M_g[r][j]); slot 2G-2 holds the scan's copy of
// the start state, so pass 3 never reads S0 while S_out (which may alias it)
// is being written.
__device__ __forceinline__ float* map_slot(float* maps, int bh, int G, int idx) {
  return maps + (size_t(bh) * (2 * G - 1) + idx) * size_t(D) * D;
}

// X^T Tx^T for X = K (Tx = T', negated: -W^T) or V (Tx = T'': U'^T) with the
// record's operand tiles (in LDS at tiles, lane's 16 bytes at lane * 16):
// out[mi][ib] holds channels 16(2w + mi) + 4g + e of token 16ib + l16 (C layout).
__device__ __forceinline__ void tproduct(const uint4* X, const unsigned char* tiles, bool negate, int wave, int lane,
                                         int g, int l16, bf16x4 (&out)[2][4]) {
  bf16x8 tb[kRecTiles];
#pragma unroll
  for (int t = 0; t < kRecTiles; ++t) tb[t] = *reinterpret_cast<const bf16x8*>(tiles + t * 1024 + lane * 16);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int colb = 16 * (2 * wave + mi) + 4 * (l16 & 3);
    bf16x8 xa[2];
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      const int jr = 32 * js + 8 * g + (l16 >> 2);
      xa[js] = join(ld4_tr(X, jr, colb), ld4_tr(X, jr + 4, colb));
    }
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < 2; ++js)
        if (32 * js <= 16 * ib + 15) w = mfma16(xa[js], tb[rec_tile(js, ib)], w);
      out[mi][ib] = to_bf16x4(negate ? -w : w);
    }
  }
}

// OUT = true: pass 3 (outputs, from the segment's true start state).
// OUT = false: pass 1; blockIdx.x = g: the workgroup runs two chains over the
// segment's chunks, from S = 0 with the value term (end state N_g) and from
// S = I without it (end state M_g, each state row r being row r of the product
// of the chunks' M_c). Both read the same tiles, W and K^T operands, so one
// workgroup holding both states (one round of workgroups on the chip instead
// of two) forms those once per chunk.
template <bool OUT, typename Tout>
__global__ void __launch_bounds__(NT, 2)
gdn_seg_kernel(GdnParams p, int G, int seg_chunks, float* maps, const unsigned char* recs) {
  __shared__ __attribute__((aligned(16))) uint4 K0[TILE];
  __shared__ __attribute__((aligned(16))) uint4 K1[OUT ? 1 : TILE];   // pass 1: K double-buffered
  __shared__ __attribute__((aligned(16))) uint4 Vt[TILE];
  __shared__ __attribute__((aligned(16))) uint4 R1[TILE];
  __shared__ __attribute__((aligned(16))) uint4 Qt[OUT ? TILE : 1];
  __shared__ __attribute__((aligned(16))) uint4 XA[OUT ? C * QP * 2 / 16 : 1];
  __shared__ SegVec sv;
  const int h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int seg = int(blockIdx.x);
  const int bh = b * p.H + h;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int col0 = 32 * wave;   // this wave's state columns
  const size_t HD = size_t(p.H) * D;
  const unsigned tok_bytes = unsigned(HD * sizeof(bf16));
  int c0, c1;
  seg_range(seg, seg_chunks, p.n_chunks, c0, c1);
  bf16 (*aqk)[QP] = reinterpret_cast<bf16 (*)[QP]>(XA);

  // ---- start state (pass 1: S the N chain's, SM the M chain's) ----
  State S, SM;
  {
    const int lane = int(threadIdx.x) & 63, g = lane >> 4, l16 = lane & 15;
    const float* src = nullptr;
    if (OUT) src = G == 1 ? p.S0 : map_slot(maps, bh, G, seg == 0 ? 2 * G - 2 : 2 * (seg - 1));
    const size_t sbase = OUT && G == 1 ? size_t(bh) * D * D : 0;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = col0 + 16 * nb + l16, row = 16 * mb + 4 * g;
        f32x4 v = {0.f, 0.f, 0.f, 0.f}, vm = {0.f, 0.f, 0.f, 0.f};
        if (src) {
          const float4 x = *reinterpret_cast<const float4*>(src + sbase + size_t(col) * D + row);
          v = f32x4{x.x, x.y, x.z, x.w};
        }
        if (!OUT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) vm[e] = row + e == col ? 1.f : 0.f;
        }
        S.st[mb][nb] = v;
        SM.st[mb][nb] = vm;
      }
  }
  const unsigned char* kg = static_cast<const unsigned char*>(p.k);
  const unsigned char* qg = static_cast<const unsigned char*>(p.q);
  const unsigned char* vg = static_cast<const unsigned char*>(p.v);
  // Buffer resources over this (batch row, head)'s token rows of k, q, v
  // (tok_bytes apart; offsets past the last token read as zeros, which the
  // ragged last chunk relies on) and over its records. The per-lane offsets
  // of the tile slots are fixed here; each chunk adds a scalar offset.
  const size_t org = (size_t(b) * p.L * HD + size_t(h) * D) * sizeof(bf16);
  const size_t span = size_t(p.L - 1) * tok_bytes + D * sizeof(bf16);
  const __amdgpu_buffer_rsrc_t rsk = make_rsrc(kg + org, span), rsq = make_rsrc(qg + org, span),
                               rsv = make_rsrc(vg + org, span);
  const __amdgpu_buffer_rsrc_t rsr = make_rsrc(recs + size_t(bh) * p.n_chunks * kRecBytes,
                                               size_t(p.n_chunks) * kRecBytes);
  // Each chunk's outputs are stored after the next chunk's loads have been
  // waited for: the wait counts stores too, and a store just issued would
  // hold it up. out_pend holds them meanwhile (rows < pend_n of token pend_t0 ..).
  typedef typename std::conditional<sizeof(Tout) == 2, bf16x4, f32x4>::type OutVec;
  OutVec out_pend[4][2];
  long long pend_t0 = 0;
  int pend_n = 0;
  unsigned char* obase = reinterpret_cast<unsigned char*>(static_cast<Tout*>(p.o) + size_t(b) * p.L * HD +
                                                          size_t(h) * D + col0);
  auto store_pending = [&](int l16, int g) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int row = 16 * tb + l16;
        if (row < pend_n) {
          const unsigned off = (unsigned(pend_t0 + row) * unsigned(HD) + unsigned(16 * nb + 4 * g)) * sizeof(Tout);
          *reinterpret_cast<OutVec*>(obase + off) = out_pend[tb][nb];
        }
      }
    pend_n = 0;
  };

  // direct loads of chunk ch's rows of one tensor into a tile, and of its
  // record into R1 (each wave its share of the 16-byte slots)
  // (the per-lane source offsets are formed at each use from a lane index
  // the compiler cannot carry across the loop, rather than kept live in
  // registers beside the state)
  auto load_rows = [&](__amdgpu_buffer_rsrc_t rs, uint4* tile, int ch) __attribute__((always_inline)) {
    const unsigned soff = unsigned((long long)ch * C) * tok_bytes;
    int lane = int(threadIdx.x) & 63;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int j = wave + 4 * i;
      if (j < PQ) {
        const int P = 64 * j + lane, row = P / PQ, c16 = P - row * PQ;   // tile slot P: row, 16-byte column
        dma16r(rs, unsigned(row) * tok_bytes + unsigned(c16 > 15 ? 15 : c16) * 16u, soff, &tile[64 * j]);
      }
    }
  };
  auto load_record = [&](int ch) __attribute__((always_inline)) {
    const int lane = int(threadIdx.x) & 63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = wave + 4 * i;   // 1 KB piece k of the record
      if (k < (kRecBytes + 1023) / 1024)
        dma16r(rsr, unsigned(lane) * 16u, unsigned(ch) * kRecBytes + 1024u * k, &R1[64 * k]);
    }
  };
  // The first chunk's tiles; every later chunk's are issued during the chunk
  // before it, each as soon as that chunk is done with the tile: V and the
  // record after U, Q after the outputs, K after the state update (pass 3;
  // pass 1 has LDS to spare for a second K tile, so there the next chunk's K
  // is issued before this one's chain).
  if (c0 < c1) {
    load_rows(rsk, K0, c0);
    if (OUT) load_rows(rsq, Qt, c0);
    load_rows(rsv, Vt, c0);
    load_record(c0);
  }
  int pf = 0;   // value of the L2 prefetch load (never used)
  // One chunk with its K in Kt (pass 1: the next chunk's K goes to Kn). The
  // loop below is unrolled by two for pass 1 so that each step names its
  // buffers directly (the compiler tracks the loads into each by name).
  auto chunk_step = [&](int chunk, uint4* Kt, uint4* Kn) __attribute__((always_inline)) {
    // The thread index passes through an empty asm each chunk, so per-lane
    // addresses are recomputed here instead of being hoisted out of the loop
    // (dozens of them would stay live across it, beside the state).
    int tid = int(threadIdx.x);
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const long long t0 = (long long)chunk * C;
    const int n = int(p.L - t0 < C ? p.L - t0 : C);

    wait_vmem();   // this chunk's tiles (and the previous chunk's stores and prefetch)
    // the prefetch value is consumed here, where the wait above has covered
    // it, so the compiler adds no wait of its own for it
    asm volatile("" ::"v"(pf));
    if (OUT) store_pending(l16, g);
    // L2 prefetch of the next chunk's k rows (one 4-byte load per 128-byte
    // line into a register): their tile is loaded last, after this chunk's
    // state update
    if (OUT && chunk + 1 < c1 && wave < 2)
      pf = __builtin_amdgcn_raw_buffer_load_b32(   // line 64 wave + lane = token * 2 + half
          rsk, unsigned(32 * wave + (lane >> 1)) * tok_bytes + 128u * unsigned(lane & 1), unsigned(t0 + C) * tok_bytes,
          0);
    lds_barrier();   // every wave's share of the tiles is in
    // ---- per-token scales from the record (and, pass 3, the query norms: 4 threads per row) ----
    const float* rec_g = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(R1) + kRecG);
    const float* rec_rk = reinterpret_cast<const float*>(reinterpret_cast<const unsigned char*>(R1) + kRecRk);
    {
      const int row = tid >> 2, part = tid & 3;
      float rq = 1.f;
      if (OUT) {
        float s2q = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 qv = ld8(Qt, row, 32 * part + 8 * c);
#pragma unroll
          for (int e = 0; e < 8; ++e) s2q += static_cast<float>(qv[e]) * static_cast<float>(qv[e]);
        }
        s2q += __shfl_xor(s2q, 1, 4);
        s2q += __shfl_xor(s2q, 2, 4);
        rq = p.l2norm ? 1.f / sqrtf(s2q + kL2Eps) : 1.f;
      }
      if (part == 0) {
        const float gi = rec_g[row], gl = rec_g[C - 1];
        if (OUT) {
          sv.rq[row] = rq;
          sv.sq[row] = row < n ? __expf(gi) * rq : 0.f;             // rows of Q S^T
        }
        sv.sk[row] = row < n ? __expf(gl - gi) * rec_rk[row] : 0.f;  // rows of U in the update
        if (row == 0) sv.gC = __expf(gl);
      }
    }
    lds_barrier();
    // ---- Aqk (pass 3): exp(g_i - g_j) q^_i.k^_j, j <= i; wave w owns rows 16w .. ----
    if (OUT) {
      bf16x8 aq[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) aq[ks] = ld8(Qt, 16 * wave + l16, 32 * ks + 8 * g);
      float gi[4], rqi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * wave + 4 * g + e;
        gi[e] = rec_g[i];
        rqi[e] = sv.rq[i];
      }
      // all four column blocks (the ones above the diagonal are masked to 0):
      // four independent product chains instead of up to four in sequence
      f32x4 qkb[4];
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) qkb[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) qkb[jb] = mfma16(aq[ks], ld8(Kt, 16 * jb + l16, 32 * ks + 8 * g), qkb[jb]);
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const f32x4 qk = qkb[jb];
        const int j = 16 * jb + l16;
        const float gj = rec_g[j], rj = rec_rk[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * wave + 4 * g + e;
          aqk[i][j] = static_cast<bf16>(j <= i ? __expf(gi[e] - gj) * rqi[e] * rj * qk[e] : 0.f);
        }
      }
    }
    // ---- -W^T = -K^T T'^T and U'^T = V^T T''^T (wave w: channel blocks 2w, 2w+1) ----
    bf16x4 wkeep[2][4], ukeep[2][4];
    {
      const unsigned char* rec = reinterpret_cast<const unsigned char*>(R1);
      tproduct(Kt, rec + kRecTp, true, wave, lane, g, l16, wkeep);
      tproduct(Vt, rec + kRecTpp, false, wave, lane, g, l16, ukeep);
    }
    lds_barrier();   // V is read: -W goes to R1, U' over V
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        // C layout: column = token 16ib + l16, rows = channels 16(2w + mi) + 4g + e
        const int tok = 16 * ib + l16, ch = 16 * (2 * wave + mi) + 4 * g;
        st4(R1, tok, ch, wkeep[mi][ib]);
        st4(Vt, tok, ch, ukeep[mi][ib]);
      }
    lds_barrier();
    // pass 1: the next chunk's K into the other buffer (it held the previous
    // chunk's K; issued after this chunk's LDS stores, which the compiler
    // would otherwise hold behind it)
    if (!OUT && chunk + 1 < c1) load_rows(rsk, Kn, chunk + 1);

    // ---- chain: U = U' - W S^T, outputs, state update (wave w: state columns 32w ..) ----
    // U of one state (with U' when the value term takes part); sb its bf16 copy
    auto chain_u = [&](const State& St, bool values, bf16x8 (&sb)[2][4], f32x4 (&u)[4][2])
        __attribute__((always_inline)) {
      state_bf16(St, sb);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          if (values) {
            const bf16x4 up = ld4_tr(Vt, 16 * tb + 4 * g + (l16 >> 2), col0 + 16 * nb + 4 * (l16 & 3));
            u[tb][nb] = f32x4{static_cast<float>(up[0]), static_cast<float>(up[1]), static_cast<float>(up[2]),
                              static_cast<float>(up[3])};
          } else {
            u[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        bf16x8 aw[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          aw[ks] = join(ld4(R1, 16 * tb + l16, 32 * ks + 4 * g), ld4(R1, 16 * tb + l16, 32 * ks + 16 + 4 * g));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) u[tb][nb] = mfma16(aw[ks], sb[nb][ks], u[tb][nb]);
      }
    };
    // S^T <- gamma_C S^T + K^T diag(sk) U
    auto chain_update = [&](State& St, const f32x4 (&u)[4][2]) __attribute__((always_inline)) {
      bf16x8 usb[2][2];
#pragma unroll
      for (int js = 0; js < 2; ++js) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sv.sk[32 * js + 4 * g]);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sv.sk[32 * js + 16 + 4 * g]);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          usb[nb][js] = join(to_bf16x4(u[2 * js][nb] * s0), to_bf16x4(u[2 * js + 1][nb] * s1));
      }
      const float gc = sv.gC;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        bf16x8 ak[2];
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          const int col = 16 * mb + 4 * (l16 & 3);
          ak[js] = join(ld4_tr(Kt, 32 * js + 4 * g + (l16 >> 2), col),
                        ld4_tr(Kt, 32 * js + 16 + 4 * g + (l16 >> 2), col));
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) St.st[mb][nb][e] *= gc;
#pragma unroll
          for (int js = 0; js < 2; ++js) St.st[mb][nb] = mfma16(ak[js], usb[nb][js], St.st[mb][nb]);
        }
      }
    };
    bf16x8 sb[2][4];
    f32x4 u[4][2];
    if constexpr (!OUT) {
      // the N chain's whole step, then the M chain's U (K stays in its
      // buffer for the whole chunk: the next chunk's K went to the other one)
      chain_u(S, true, sb, u);
      chain_update(S, u);
      chain_u(SM, false, sb, u);
    } else {
      chain_u(S, true, sb, u);
    }
    lds_barrier();   // every wave has read U' (over V) and -W (in R1)
    if (chunk + 1 < c1) {
      load_rows(rsv, Vt, chunk + 1);
      load_record(chunk + 1);
    }
    if (OUT) {
      // O^T = S Q^T diag(sq) + U^T Aqk^T: lane holds channels col0 + 16nb + 4g + e of token 16tb + l16
      bf16x8 ub[2][2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int js = 0; js < 2; ++js) ub[nb][js] = join(to_bf16x4(u[2 * js][nb]), to_bf16x4(u[2 * js + 1][nb]));
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int row = 16 * tb + l16;
        bf16x8 aq[4], aa[2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          aq[ks] = join(ld4(Qt, row, 32 * ks + 4 * g), ld4(Qt, row, 32 * ks + 16 + 4 * g));
#pragma unroll
        for (int js = 0; js < 2; ++js)
          aa[js] = join(*reinterpret_cast<const bf16x4*>(&aqk[row][32 * js + 4 * g]),
                        *reinterpret_cast<const bf16x4*>(&aqk[row][32 * js + 16 + 4 * g]));
        const float sqv = sv.sq[row];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) x = mfma16(sb[nb][ks], aq[ks], x);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= sqv;
#pragma unroll
          for (int js = 0; js < 2; ++js)
            if (32 * js <= 16 * tb + 15) x = mfma16(ub[nb][js], aa[js], x);
          pend_t0 = t0;
          pend_n = n;
          if constexpr (sizeof(Tout) == 2) {
            out_pend[tb][nb] = to_bf16x4(x);
          } else {
            out_pend[tb][nb] = x;
          }
        }
      }
    }
    if (OUT) {
      lds_barrier();   // every wave has read Q and Aqk
      if (chunk + 1 < c1) load_rows(rsq, Qt, chunk + 1);
    }
    chain_update(OUT ? S : SM, u);
    if (OUT) {
      lds_barrier();   // every wave has read K
      if (chunk + 1 < c1) load_rows(rsk, Kt, chunk + 1);
    }
  };
  if constexpr (OUT) {
    for (int chunk = c0; chunk < c1; ++chunk) chunk_step(chunk, K0, K0);
  } else {
    for (int chunk = c0; chunk < c1; chunk += 2) {
      chunk_step(chunk, K0, K1);
      if (chunk + 1 < c1) chunk_step(chunk + 1, K1, K0);
    }
  }

  if (OUT) {
    const int lane = int(threadIdx.x) & 63;
    store_pending(lane & 15, lane >> 4);
  }
  // ---- end state: S^T tile (mb, nb) holds rows d_k 16mb + 4g + e of state row col0 + 16nb + l16 ----
  auto store_state = [&](const State& St, float* dst, bool transposed) {
    const int lane = int(threadIdx.x) & 63, g = lane >> 4, l16 = lane & 15;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int r = col0 + 16 * nb + l16, j = 16 * mb + 4 * g;
        if (!transposed) {
          *reinterpret_cast<float4*>(dst + size_t(r) * D + j) =
              make_float4(St.st[mb][nb][0], St.st[mb][nb][1], St.st[mb][nb][2], St.st[mb][nb][3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[size_t(j + e) * D + r] = St.st[mb][nb][e];
        }
      }
  };
  if (OUT) {
    if (seg == G - 1 && p.S_out) store_state(S, p.S_out + size_t(bh) * D * D, false);
  } else {
    store_state(S, map_slot(maps, bh, G, 2 * seg), false);
    store_state(SM, map_slot(maps, bh, G, 2 * seg + 1), true);
  }
}

// ---------------------------------------------------------------------------
// pass 2: S_{g+1} = S_g M_g + N_g over the segments of one head
// ---------------------------------------------------------------------------
// One workgroup per (16 state rows, head, batch row); wave w computes the
// transposed product S_{g+1}^T = M_g^T S_g^T + N_g^T for d_k rows 32w ..
// 32w+31. Products in bf16 MFMA with both factors split into a high and a
// low bf16 part (x = hi + lo): hi*hi + hi*lo + lo*hi, fp32 accumulation, so
// the result keeps about 16 significant bits per factor. The next segment's
// M and N are loaded while the current product runs.
constexpr int kScanRows = 16;
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = static_cast<bf16>(x[e]);
    lo[e] = static_cast<bf16>(x[e] - static_cast<float>(hi[e]));
  }
}

struct ScanOperands {
  float4 m[2][4][2];   // M^T rows of this wave's two tiles, permuted d_k pairs
  float4 nv[2];        // N^T start values (C layout)
};

__device__ __forceinline__ void scan_load(ScanOperands& x, float* maps, int bh, int G, int s, int r0, int wave,
                                          int g, int l16) {
  const float* Nslot = map_slot(maps, bh, G, 2 * s);
  const float* Mt = map_slot(maps, bh, G, 2 * s + 1);
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int j0 = 32 * wave + 16 * t;
    x.nv[t] = *reinterpret_cast<const float4*>(Nslot + size_t(r0 + l16) * D + j0 + 4 * g);
    const float* mrow = Mt + size_t(j0 + l16) * D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      x.m[t][ks][0] = *reinterpret_cast<const float4*>(mrow + 32 * ks + 4 * g);
      x.m[t][ks][1] = *reinterpret_cast<const float4*>(mrow + 32 * ks + 16 + 4 * g);
    }
  }
}

__global__ void __launch_bounds__(NT)
gdn_seg_scan(GdnParams p, int G, float* maps) {
  __shared__ __attribute__((aligned(16))) float Ssh[kScanRows][D + 4];
  const int rb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  if (skipped(p.skip, b)) return;
  const int bh = b * p.H + h;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = tid >> 6;
  const int r0 = kScanRows * rb;   // state rows r0 .. r0+15
  ScanOperands cur, nxt;
  scan_load(cur, maps, bh, G, 0, r0, wave, g, l16);
  // S_0 rows into LDS and into the start-state copy that pass 3 reads
  float* S0copy = map_slot(maps, bh, G, 2 * G - 2);
  for (int i = tid; i < kScanRows * D; i += NT) {
    const int r = i / D, c = i % D;
    const float x = p.S0 ? p.S0[size_t(bh) * D * D + size_t(r0 + r) * D + c] : 0.f;
    Ssh[r][c] = x;
    S0copy[size_t(r0 + r) * D + c] = x;
  }
  __syncthreads();
  for (int s = 0; s + 1 < G; ++s) {
    if (s + 2 < G) scan_load(nxt, maps, bh, G, s + 1, r0, wave, g, l16);
    // B operand: S_g^T (k = state column r, permuted), column = state row l16
    bf16x8 bh_[4], bl_[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = Ssh[l16][32 * ks + 4 * g + e];
        x[4 + e] = Ssh[l16][32 * ks + 16 + 4 * g + e];
      }
      split8(x, bh_[ks], bl_[ks]);
    }
    f32x4 acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // C layout: rows d_k 32w + 16t + 4g + e, column = state row r0 + l16; starts from N^T
      acc[t] = f32x4{cur.nv[t].x, cur.nv[t].y, cur.nv[t].z, cur.nv[t].w};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const float4 m0 = cur.m[t][ks][0], m1 = cur.m[t][ks][1];
        const float x[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        bf16x8 ah, al;
        split8(x, ah, al);
        acc[t] = mfma16(ah, bh_[ks], acc[t]);
        acc[t] = mfma16(ah, bl_[ks], acc[t]);
        acc[t] = mfma16(al, bh_[ks], acc[t]);
      }
    }
    __syncthreads();   // every wave has read S_g
    float* Nslot = map_slot(maps, bh, G, 2 * s);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = 32 * wave + 16 * t + 4 * g;
      *reinterpret_cast<float4*>(&Ssh[l16][j]) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
      // S_{g+1} over N_g: pass 3 of segment g + 1 starts from it
      *reinterpret_cast<float4*>(Nslot + size_t(r0 + l16) * D + j) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
    __syncthreads();
    cur = nxt;
  }
}

}  // namespace

hipError_t launch_gdn_seg(const GdnParams& p, int G, int seg_chunks, void* workspace, int out_dt, hipStream_t st) {
  unsigned char* recs = static_cast<unsigned char*>(workspace);
  float* maps = reinterpret_cast<float*>(recs + gdn_seg_record_bytes(p.B, p.H, p.n_chunks));
  hipLaunchKernelGGL(gdn_tinv_kernel, dim3(p.n_chunks, p.H, p.B), dim3(NT), 0, st, p, recs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (G > 1) {
    hipLaunchKernelGGL((gdn_seg_kernel<false, bf16>), dim3(G - 1, p.H, p.B), dim3(NT), 0, st, p, G,
                       seg_chunks, maps, recs);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn_seg_scan, dim3(D / kScanRows, p.H, p.B), dim3(NT), 0, st, p, G, maps);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (out_dt == HLTA_BF16)
    hipLaunchKernelGGL((gdn_seg_kernel<true, bf16>), dim3(G, p.H, p.B), dim3(NT), 0, st, p, G, seg_chunks, maps,
                       recs);
  else
    hipLaunchKernelGGL((gdn_seg_kernel<true, float>), dim3(G, p.H, p.B), dim3(NT), 0, st, p, G, seg_chunks, maps,
                       recs);
  return hipGetLastError();
}

}  // namespace hlta
