// Backward of the softmax branches (SWA + DSWA) with bf16 MFMA on gfx950:
// bf16 q, k, v and upstream gradient, d = 128, P >= 64, fp32 gradients.
//
// The branches are exact softmax attention over each query frame's key set
// (Kairos abstract, point (2)); their gradient is the textbook one, computed
// tile by tile with the scores recomputed on chip (long-context page, section
// 03 on tiled exact attention). With s = scale, c = s * log2(e), per branch i
// with mix weight w_i (dO = w_i * d_mix):
//   lse_q  = log2 sum_k exp2(c q.k)                       (row statistics pass)
//   D_q    = w_i * d_mix_q . o_q   (o as the forward stored it)
//   P_qk   = exp2(c q.k - lse_q),  dS_qk = P_qk (w_i d_mix_q . v_k - D_q)
//   dq_q   = s sum_k dS_qk k_k                            (query-major pass)
//   dk_k   = s sum_q dS_qk q_q,  dv_k = sum_q w_i P_qk d_mix_q (key-major pass)
// summed over both branches. Four kernels on the caller's stream; statistics
// are kept [branch][b][h][token] so a tile's rows are contiguous.
//
// The query-major pass is the forward kernel's layout (scores transposed,
// S^T = K Q^T, so a lane holds 32 key scores of one query, which is the
// B-operand layout of the next product): dP^T = V dO^T uses the V rows the
// way S^T uses the K rows, and dQ^T += K^T dS^T reads K transposed the way the
// forward reads V^T. The key-major pass swaps the roles: a wave keeps 32 key
// rows (K and V) in registers, streams the queries (and d_mix rows) of the
// frames that read its key frame through LDS, computes X = Q K^T and
// dP = dO V^T (a lane holds one key's column), and accumulates
// dV^T += dO^T (w P) and dK^T += Q^T dS with transposed tile reads.
#include "attn_mfma_tiles.h"
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int RT = 128;   // rows (queries or keys) per workgroup: 4 waves x 32

// Work item n (XCD-aware order as in the forward): row tile, frame, (b, h).
struct Item {
  int rt, f, b, h;
};
__device__ __forceinline__ bool item_of(const AttnParams& p, Item& it) {
  const int nrt = (p.P + RT - 1) / RT;
  const long long total = (long long)p.B * p.H * p.T * nrt;
  const long long per_xcd = (total + kXcds - 1) / kXcds;
  const long long n = (long long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (n >= total) return false;
  it.rt = int(n % nrt);
  const long long rest = n / nrt;
  it.f = p.T - 1 - int(rest % p.T);
  const int bh = int(rest / p.T);
  it.b = bh / p.H;
  it.h = bh % p.H;
  return true;
}

unsigned grid_of(const AttnParams& p) {
  const long long nrt = (p.P + RT - 1) / RT;
  const long long total = (long long)p.B * p.H * p.T * nrt;
  return unsigned((total + kXcds - 1) / kXcds * kXcds);
}

// 8 chunks (one 32-row MFMA operand set) of row `row` of a [.., H, D] bf16 tensor
__device__ __forceinline__ void load_rows(const bf16* base, int row, bool ok, size_t HD, int hl, bf16x8 (&v)[8]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ok) u = *reinterpret_cast<const uint4*>(base + size_t(row) * HD + ks * 16 + hl * 8);
    v[ks] = *reinterpret_cast<bf16x8*>(&u);
  }
}

__device__ __forceinline__ void dma_offsets(int wave, int lane, size_t ts, unsigned (&off)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + (lane >> 4);
    off[j] = unsigned(row) * unsigned(ts * sizeof(bf16)) + unsigned(swz(row, lane & 15)) * 16u;
  }
}

// store the 32 x 128 tile held transposed in acc (lane: row l32, d = db*32 + 8j + 4hl + e) times f
__device__ __forceinline__ void store_rows(float* dst, const f32x16 (&acc)[4], float f, int hl) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = acc[db][4 * j + e] * f;
      store4(dst + db * 32 + j * 8 + 4 * hl, o4);
    }
}

// ---------------------------------------------------------------------------
// row statistics: lse_q (log2 units) per branch, from S^T = K Q^T tiles
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(NT, 2) attn_bwd_lse_mfma(AttnParams p, float* lse) {
  __shared__ Tile sK0, sK1;
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, hl = lane >> 5, l32 = lane & 31;
  Item it;
  if (!item_of(p, it)) return;
  const long long f = it.f;
  const size_t HD = size_t(p.H) * D;
  const int qrow = it.rt * RT + wave * 32 + l32;
  const bool wave_active = it.rt * RT + wave * 32 < p.P;
  const size_t fbase = ((size_t(it.b) * p.T + it.f) * p.P) * HD + size_t(it.h) * D;
  bf16x8 qv[8];
  load_rows(static_cast<const bf16*>(p.q) + fbase, qrow, qrow < p.P, HD, hl, qv);
  unsigned off[4];
  dma_offsets(wave, lane, HD, off);
  KeyStream<false> kst;
  kst.fstride = size_t(p.P) * HD;
  kst.P = p.P;
  kst.kmain = uni(static_cast<const bf16*>(p.k) + size_t(it.b) * p.T * kst.fstride + size_t(it.h) * D);
  kst.vmain = kst.kmain;
  const float c = p.scale_log2;
  const int nswa = swa_count(f, p.W), ndswa = dswa_count(f, p.dil, p.taps);
  const size_t L = size_t(p.T) * p.P;
  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    const int ntiles = int((nk + KT - 1) / KT);
    float m = -INFINITY, lsum = 0.f;
    KeyStream<false> ks = kst;
    ks.start(branch == 0 ? f - nswa + 1 : f - p.dil, branch == 0 ? 1 : -p.dil, nframes);
    __syncthreads();
    auto kleft_of = [&](int t) {
      const long long left = nk - (long long)t * KT;
      return int(left < KT ? (left > 0 ? left : 0) : KT);
    };
    if (ntiles > 0) issue_tile<false, false>(sK0, sK0, ks, kleft_of(0), off, HD, wave, lane);
    auto tile = [&](int t, const Tile& Kt, Tile& Kn) __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();
      if (t + 1 < ntiles) {
        ks.advance();
        issue_tile<false, false>(Kn, Kn, ks, kleft_of(t + 1), off, HD, wave, lane);
      }
      if (wave_active) {
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_chunk(Kt, kb, l32, 2 * k8 + hl), qv[k8], s[kb], 0,
                                                             0, 0);
        }
        const int kthr = uni(kleft_of(t)) - 4 * hl;
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (kb * 32 + (r >> 2) * 8 + (r & 3) >= kthr) s[kb][r] = -INFINITY;
            mt = fmaxf(mt, s[kb][r]);
          }
        mt = max_xor32(mt) * c;
        const float mn = fmaxf(m, mt);
        float acc = lsum * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mn));
        lsum = acc;
        m = mn;
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, sK0, sK1);
      if (t + 1 < ntiles) tile(t + 1, sK1, sK0);
    }
    if (wave_active && ntiles > 0) {
      const float ltot = sum_xor32(lsum);
      if (hl == 0 && qrow < p.P)
        lse[((size_t(branch) * p.B + it.b) * p.H + it.h) * L + size_t(it.f) * p.P + qrow] = m + log2f(ltot);
    }
  }
}

// ---------------------------------------------------------------------------
// D = w_i * d_mix . o_i per (token, head) and branch; 16 lanes per row
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) attn_bwd_dsum(const bf16* g, const bf16* o_swa, const bf16* o_dswa,
                                                     const float* mix_w, float* dsum, int B, long long L, int H) {
  const long long rows = (long long)B * L * H;
  const int sub = threadIdx.x & 15;
  for (long long r = (long long)blockIdx.x * 16 + (threadIdx.x >> 4); r < rows; r += (long long)gridDim.x * 16) {
    const size_t e = size_t(r) * D + sub * 8;
    const uint4 ug = *reinterpret_cast<const uint4*>(g + e);
    const uint4 u0 = *reinterpret_cast<const uint4*>(o_swa + e);
    const uint4 u1 = *reinterpret_cast<const uint4*>(o_dswa + e);
    const bf16* pg = reinterpret_cast<const bf16*>(&ug);
    const bf16* p0 = reinterpret_cast<const bf16*>(&u0);
    const bf16* p1 = reinterpret_cast<const bf16*>(&u1);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = static_cast<float>(pg[i]);
      s0 += x * static_cast<float>(p0[i]);
      s1 += x * static_cast<float>(p1[i]);
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      s0 += __shfl_xor(s0, o, 16);
      s1 += __shfl_xor(s1, o, 16);
    }
    if (sub == 0) {
      const int h = int(r % H);
      const long long bt = r / H;
      const int b = int(bt / L);
      const long long t = bt % L;
      dsum[(size_t(b) * H + h) * L + t] = mix_w[3 * h] * s0;
      dsum[((size_t(B) + b) * H + h) * L + t] = mix_w[3 * h + 1] * s1;
    }
  }
}

// ---------------------------------------------------------------------------
// dq, query-major
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(NT, 2)
attn_bwd_dq_mfma(AttnParams p, const bf16* g, const float* mix_w, const float* lse, const float* dsum, float* dq,
                 float scale) {
  __shared__ Tile sK0, sV0, sK1, sV1;
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, hl = lane >> 5, l32 = lane & 31, l16 = lane & 15;
  Item it;
  if (!item_of(p, it)) return;
  const long long f = it.f;
  const size_t HD = size_t(p.H) * D;
  const int qrow = it.rt * RT + wave * 32 + l32;
  const bool qok = qrow < p.P;
  const bool wave_active = it.rt * RT + wave * 32 < p.P;
  const size_t fbase = ((size_t(it.b) * p.T + it.f) * p.P) * HD + size_t(it.h) * D;
  bf16x8 qv[8], gv[8];
  load_rows(static_cast<const bf16*>(p.q) + fbase, qrow, qok, HD, hl, qv);
  load_rows(g + fbase, qrow, qok, HD, hl, gv);
  unsigned off[4];
  dma_offsets(wave, lane, HD, off);
  KeyStream<false> kst;
  kst.fstride = size_t(p.P) * HD;
  kst.P = p.P;
  const size_t o = size_t(it.b) * p.T * kst.fstride + size_t(it.h) * D;
  kst.kmain = uni(static_cast<const bf16*>(p.k) + o);
  kst.vmain = uni(static_cast<const bf16*>(p.v) + o);
  const float c = p.scale_log2;
  const int nswa = swa_count(f, p.W), ndswa = dswa_count(f, p.dil, p.taps);
  const size_t L = size_t(p.T) * p.P;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    const int ntiles = int((nk + KT - 1) / KT);
    const float w = mix_w[3 * it.h + branch];
    const size_t si = ((size_t(branch) * p.B + it.b) * p.H + it.h) * L + size_t(it.f) * p.P + (qok ? qrow : 0);
    const float lq = (qok && ntiles > 0) ? lse[si] : 0.f;
    const float dq_ = qok ? dsum[si] : 0.f;
    KeyStream<false> ks = kst;
    ks.start(branch == 0 ? f - nswa + 1 : f - p.dil, branch == 0 ? 1 : -p.dil, nframes);
    __syncthreads();
    auto kleft_of = [&](int t) {
      const long long left = nk - (long long)t * KT;
      return int(left < KT ? (left > 0 ? left : 0) : KT);
    };
    if (ntiles > 0) issue_tile(sK0, sV0, ks, kleft_of(0), off, HD, wave, lane);
    auto tile = [&](int t, const Tile& Kt, const Tile& Vt, Tile& Kn, Tile& Vn) __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();
      if (t + 1 < ntiles) {
        ks.advance();
        issue_tile(Kn, Vn, ks, kleft_of(t + 1), off, HD, wave, lane);
      }
      if (wave_active) {
        const int kthr = uni(kleft_of(t)) - 4 * hl;
        bf16x8 dsb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_chunk(Kt, kb, l32, 2 * k8 + hl), qv[k8], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_chunk(Vt, kb, l32, 2 * k8 + hl), gv[k8], dp, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lq));
            if (kb * 32 + (r >> 2) * 8 + (r & 3) >= kthr) pr = 0.f;
            dsb[kb][r >> 3][r & 7] = static_cast<bf16>(pr * fmaf(w, dp[r], -dq_));
          }
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_vt(Kt, kb, m2, hl, db * 32 + (l32 & 16), l16),
                                                                dsb[kb][m2], acc[db], 0, 0, 0);
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, sK0, sV0, sK1, sV1);
      if (t + 1 < ntiles) tile(t + 1, sK1, sV1, sK0, sV0);
    }
  }
  if (qok) store_rows(dq + fbase + size_t(qrow) * HD, acc, scale, hl);
}

// ---------------------------------------------------------------------------
// dk, dv, key-major: the wave's 32 key rows stay in registers; the query rows
// (and d_mix rows) of the frames that read this key frame stream through LDS
// ---------------------------------------------------------------------------
// token index (in the batch row) of query j of the tile at the stream's position
__device__ __forceinline__ long long tile_token(const KeyStream<false>& qs, int step, int j) {
  const int split = qs.P - qs.pk;
  return j < split ? qs.g * qs.P + qs.pk + j : (qs.g + step) * qs.P + (j - split);
}

// the 64 statistics (lse and D) of a tile's query rows, global -> LDS by
// direct 4-byte loads (wave 0: lse, wave 1: D); rows past the end re-read the
// last valid row
__device__ __forceinline__ void issue_stats(float* Ld, float* Dd, const KeyStream<false>& qs, int step, int qleft,
                                            const float* lse_b, const float* ds_b, int wave, int lane) {
  if (wave > 1) return;
  const int j = lane < qleft ? lane : qleft - 1;
  const float* src = (wave == 0 ? lse_b : ds_b) + tile_token(qs, step, j);
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(wave == 0 ? Ld : Dd), 4, 0, 0);
}

// kDV: dV^T += dO^T (w P) (scores X = Q K^T only); otherwise dK^T += Q^T dS
// (X and dP = dO V^T). Two instantiations, so each holds one accumulator set
// and runs two waves per SIMD.
template <bool kDV>
__global__ void __launch_bounds__(NT, 2)
attn_bwd_dkdv_mfma(AttnParams p, const bf16* g, const float* mix_w, const float* lse, const float* dsum, float* out,
                   float scale) {
  __shared__ Tile sQ0, sG0, sQ1, sG1;
  __shared__ __attribute__((aligned(16))) float sL0[KT], sD0[KT], sL1[KT], sD1[KT];
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, hl = lane >> 5, l32 = lane & 31, l16 = lane & 15;
  Item it;
  if (!item_of(p, it)) return;
  const long long gk = it.f;   // key frame
  const size_t HD = size_t(p.H) * D;
  const int krow = it.rt * RT + wave * 32 + l32;
  const bool kok = krow < p.P;
  const bool wave_active = it.rt * RT + wave * 32 < p.P;
  const size_t fbase = ((size_t(it.b) * p.T + it.f) * p.P) * HD + size_t(it.h) * D;
  bf16x8 kv[8], vv[kDV ? 1 : 8];
  load_rows(static_cast<const bf16*>(p.k) + fbase, krow, kok, HD, hl, kv);
  if constexpr (!kDV) load_rows(static_cast<const bf16*>(p.v) + fbase, krow, kok, HD, hl, vv);
  unsigned off[4];
  dma_offsets(wave, lane, HD, off);
  KeyStream<false> qst;
  qst.fstride = size_t(p.P) * HD;
  qst.P = p.P;
  const size_t o = size_t(it.b) * p.T * qst.fstride + size_t(it.h) * D;
  qst.kmain = uni(static_cast<const bf16*>(p.q) + o);
  qst.vmain = uni(g + o);
  const float c = p.scale_log2;
  const size_t L = size_t(p.T) * p.P;
  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  for (int branch = 0; branch < 2; ++branch) {
    // query frames reading key frame gk: gk .. gk+W-1 (SWA), gk + dil*j, j = 1..taps (DSWA)
    const long long first = branch == 0 ? gk : gk + p.dil;
    const int step = branch == 0 ? 1 : p.dil;
    long long nf = branch == 0 ? (long long)p.T - gk : (p.T - 1 - gk) / p.dil;
    const int cap = branch == 0 ? p.W : p.taps;
    if (nf > cap) nf = cap;
    if (nf < 0) nf = 0;
    const int nframes = int(nf);
    const long long nq = (long long)nframes * p.P;
    const int ntiles = int((nq + KT - 1) / KT);
    const float w = mix_w[3 * it.h + branch];
    const float* lse_b = lse + ((size_t(branch) * p.B + it.b) * p.H + it.h) * L;
    const float* ds_b = dsum + ((size_t(branch) * p.B + it.b) * p.H + it.h) * L;
    KeyStream<false> qs = qst;
    qs.start(first, step, nframes);
    __syncthreads();
    auto qleft_of = [&](int t) {
      const long long left = nq - (long long)t * KT;
      return int(left < KT ? (left > 0 ? left : 0) : KT);
    };
    if (ntiles > 0) {
      issue_tile(sQ0, sG0, qs, qleft_of(0), off, HD, wave, lane);
      issue_stats(sL0, sD0, qs, step, qleft_of(0), lse_b, ds_b, wave, lane);
    }
    auto tile = [&](int t, const Tile& Qt, const Tile& Gt, const float* Lt, const float* Dt, Tile& Qn, Tile& Gn,
                    float* Ln, float* Dn) __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();
      if (t + 1 < ntiles) {
        qs.advance();
        issue_tile(Qn, Gn, qs, qleft_of(t + 1), off, HD, wave, lane);
        issue_stats(Ln, Dn, qs, step, qleft_of(t + 1), lse_b, ds_b, wave, lane);
      }
      if (wave_active) {
        const int qthr = uni(qleft_of(t)) - 4 * hl;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          f32x16 x, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = dp[r] = 0.f;
#pragma unroll
          for (int k8 = 0; k8 < 8; ++k8) {
            x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_chunk(Qt, qb, l32, 2 * k8 + hl), kv[k8], x, 0, 0, 0);
            if constexpr (!kDV)
              dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld_chunk(Gt, qb, l32, 2 * k8 + hl), vv[k8], dp, 0, 0, 0);
          }
          bf16x8 ob[2];   // w P (kDV) or dS
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            // queries qb*32 + 8 r4 + 4 hl + 0..3: their statistics as one 16-byte read each
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + qb * 32 + 8 * r4 + 4 * hl);
            f32x4 d4 = {0.f, 0.f, 0.f, 0.f};
            if constexpr (!kDV) d4 = *reinterpret_cast<const f32x4*>(Dt + qb * 32 + 8 * r4 + 4 * hl);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * r4 + e;
              float pr = __builtin_amdgcn_exp2f(fmaf(x[r], c, -l4[e]));
              if (qb * 32 + 8 * r4 + e >= qthr) pr = 0.f;
              ob[r >> 3][r & 7] = static_cast<bf16>(kDV ? w * pr : pr * fmaf(w, dp[r], -d4[e]));
            }
          }
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2)
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  ld_vt(kDV ? Gt : Qt, qb, m2, hl, db * 32 + (l32 & 16), l16), ob[m2], acc[db], 0, 0, 0);
        }
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, sQ0, sG0, sL0, sD0, sQ1, sG1, sL1, sD1);
      if (t + 1 < ntiles) tile(t + 1, sQ1, sG1, sL1, sD1, sQ0, sG0, sL0, sD0);
    }
  }
  if (kok) store_rows(out + fbase + size_t(krow) * HD, acc, kDV ? 1.f : scale, hl);
}

}  // namespace

hipError_t launch_attn_bwd_mfma(const AttnParams& p, const void* d_mix, const void* o_swa, const void* o_dswa,
                                const float* mix_w, float* lse, bool lse_given, float* dsum, float* dq, float* dk,
                                float* dv, float scale, hipStream_t st) {
  const unsigned grid = grid_of(p);
  if (grid == 0) return hipSuccess;
  const bf16* g = static_cast<const bf16*>(d_mix);
  const long long L = (long long)p.T * p.P;
  const long long rows = (long long)p.B * L * p.H;
  const unsigned dgrid = unsigned(rows / 16 + 1 < 65536 ? rows / 16 + 1 : 65536);
  if (!lse_given) hipLaunchKernelGGL(attn_bwd_lse_mfma, dim3(grid), dim3(NT), 0, st, p, lse);
  hipLaunchKernelGGL(attn_bwd_dsum, dim3(dgrid), dim3(256), 0, st, g, static_cast<const bf16*>(o_swa),
                     static_cast<const bf16*>(o_dswa), mix_w, dsum, p.B, L, p.H);
  hipLaunchKernelGGL(attn_bwd_dq_mfma, dim3(grid), dim3(NT), 0, st, p, g, mix_w, lse, dsum, dq, scale);
  hipLaunchKernelGGL(attn_bwd_dkdv_mfma<false>, dim3(grid), dim3(NT), 0, st, p, g, mix_w, lse, dsum, dk, scale);
  hipLaunchKernelGGL(attn_bwd_dkdv_mfma<true>, dim3(grid), dim3(NT), 0, st, p, g, mix_w, lse, dsum, dv, scale);
  return hipGetLastError();
}

}  // namespace hlta
