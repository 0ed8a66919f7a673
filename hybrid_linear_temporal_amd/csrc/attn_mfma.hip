// SWA + DSWA softmax attention with bf16 MFMA on gfx950 (d = 128), with the
// mix fused in the epilogue.
//
// What is computed: for every query of latent frame f, exact softmax attention
// over all keys of its frame set (SWA: frames f-W+1 .. f; DSWA: frames
// f - dil*r, r = 1..taps; Kairos abstract, point (2)), tile by tile with a
// running max and sum so the score matrix never leaves the chip (long-context
// page, section 03 on FlashAttention: every legal pair, same result, less HBM
// traffic). The keys of a branch's frames form one virtual sequence; a tile of
// 64 keys may span two frames, so every key row carries its own address.
//
// Mapping to CDNA4:
//  * workgroup = 4 waves = 128 query rows of one frame of one head; each wave
//    owns 32 query rows and keeps its Q block in registers as MFMA operand;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then holds 32 key scores of one query, which is exactly the
//    B-operand layout of O^T = V^T P^T, so P never goes through LDS;
//  * K tiles are staged in LDS key-major (16-byte rows reads), V tiles
//    transposed (d-major) so the A operand of the P.V product is two 8-byte
//    LDS reads; both are double-buffered with one barrier per tile;
//  * the softmax runs in the exp2 domain with the scale folded into one FMA;
//    row sums stay per half-wave until the epilogue;
//  * workgroups are ordered so each XCD (blockIdx mod 8) walks a contiguous
//    range of (head, frame) items, heaviest frames first: the 13 query tiles
//    of a frame and the neighbouring frames share K/V tiles in that XCD's L2.
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;        // head dim
constexpr int QT = 128;       // query rows per workgroup
constexpr int KT = 64;        // keys per tile
constexpr int NT = 256;       // threads
constexpr int KS = D + 8;     // LDS row pitch of K (bf16), 272 B
constexpr int VS = KT + 4;    // LDS row pitch of V^T (bf16), 136 B
constexpr int kXcds = 8;

struct Smem {
  bf16 K[2][KT][KS];
  bf16 Vt[2][D][VS];
};

// Staging registers of one K/V tile: each thread moves 4 K chunks of 16 B and
// a 4-key x 8-d block of V.
struct Stage {
  uint4 k[4];
  uint4 v[4];
};

// A tile of 64 consecutive keys of the virtual sequence spans at most two
// frames (P >= 64) or several (P < 64). Keys are addressed from the frame
// bases of the tile's first frame onwards; with P >= 64 the two bases are
// wave-uniform and live in scalar registers.
struct TileAddr {
  const bf16* k0;    // K row of the tile's first key
  const bf16* v0;
  const bf16* k1;    // K row 0 of the next frame (if the tile crosses into it)
  const bf16* v1;
  int split;         // keys [0, split) come from the first frame
};

__device__ __forceinline__ TileAddr tile_addr(const AttnParams& p, int b, int h, int branch, long long f,
                                              int nswa, int nframes, long long t0) {
  const bf16* km = static_cast<const bf16*>(p.k);
  const bf16* vm = static_cast<const bf16*>(p.v);
  const bf16* kr = static_cast<const bf16*>(p.ring_k);
  const bf16* vr = static_cast<const bf16*>(p.ring_v);
  const int s = int(t0 / p.P);
  const int pk = int(t0 - (long long)s * p.P);
  const long long g0 = branch_frame(branch, f, nswa, p.dil, s);
  const size_t off = size_t(pk) * p.H * D;
  TileAddr a;
  a.k0 = key_frame_ptr<bf16, D>(km, kr, p, b, h, g0) + off;
  a.v0 = key_frame_ptr<bf16, D>(vm, vr, p, b, h, g0) + off;
  a.split = p.P - pk;
  if (s + 1 < nframes) {
    const long long g1 = branch_frame(branch, f, nswa, p.dil, s + 1);
    a.k1 = key_frame_ptr<bf16, D>(km, kr, p, b, h, g1);
    a.v1 = key_frame_ptr<bf16, D>(vm, vr, p, b, h, g1);
  } else {
    a.k1 = a.k0;
    a.v1 = a.v0;
  }
  return a;
}

// row of key kk (0..63) of the tile; P >= KT assumed (at most one frame switch)
__device__ __forceinline__ const bf16* tile_row(const bf16* base0, const bf16* base1, int split, int kk,
                                                size_t tok_stride) {
  return kk < split ? base0 + size_t(kk) * tok_stride : base1 + size_t(kk - split) * tok_stride;
}

__device__ __forceinline__ void load_tile(Stage& st, const AttnParams& p, int b, int h, int branch, long long f,
                                          int nswa, int nframes, long long nk, long long t0, int tid) {
  const TileAddr ta = tile_addr(p, b, h, branch, f, nswa, nframes, t0);
  const size_t ts = size_t(p.H) * D;
  const int kleft = int(nk - t0 < KT ? nk - t0 : KT);
  // K: key = tid/16 + 16*i, 16-byte chunk c = tid%16
  const int c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = (tid >> 4) + 16 * i;
    if (kk < kleft)
      st.k[i] = *reinterpret_cast<const uint4*>(tile_row(ta.k0, ta.k1, ta.split, kk, ts) + c * 8);
    else
      st.k[i] = make_uint4(0, 0, 0, 0);
  }
  // V: keys 4*kg .. 4*kg+3, d = 8*dg .. 8*dg+7 with dg = tid%16, kg = tid/16
  const int kg = tid >> 4, dg = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int kk = 4 * kg + i;
    if (kk < kleft)
      st.v[i] = *reinterpret_cast<const uint4*>(tile_row(ta.v0, ta.v1, ta.split, kk, ts) + dg * 8);
    else
      st.v[i] = make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void store_tile(Smem& sm, int buf, const Stage& st, int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(&sm.K[buf][(tid >> 4) + 16 * i][c * 8]) = st.k[i];
  const int kg = tid >> 4, dg = tid & 15;
  // transpose the 4 x 8 block: Vt[8dg + e][4kg + i] = V[4kg + i][8dg + e]
  const unsigned short* v0 = reinterpret_cast<const unsigned short*>(&st.v[0]);
  const unsigned short* v1 = reinterpret_cast<const unsigned short*>(&st.v[1]);
  const unsigned short* v2 = reinterpret_cast<const unsigned short*>(&st.v[2]);
  const unsigned short* v3 = reinterpret_cast<const unsigned short*>(&st.v[3]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u16x4 w = {v0[e], v1[e], v2[e], v3[e]};
    *reinterpret_cast<u16x4*>(&sm.Vt[buf][8 * dg + e][4 * kg]) = w;
  }
}

__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 x = {static_cast<bf16>(v[0]), static_cast<bf16>(v[1]), static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
  *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  f32x4 x = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = x;
}
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  const bf16x4 x = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(x[e]);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = x[e];
}

template <typename Tout>
__global__ void __launch_bounds__(NT, 2)
attn_mfma_kernel(AttnParams p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hl = lane >> 5, l32 = lane & 31;

  // ---- work item (XCD-aware order, heaviest frames first) ----
  const int nqt = (p.P + QT - 1) / QT;
  const long long total = (long long)p.B * p.H * p.T * nqt;
  const long long per_xcd = (total + kXcds - 1) / kXcds;
  const long long n = (long long)(blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (n >= total) return;
  const int qt = int(n % nqt);
  const long long rest = n / nqt;
  const int fq = p.T - 1 - int(rest % p.T);
  const int bh = int(rest / p.T);
  const int b = bh / p.H, h = bh % p.H;
  const long long f = p.f0 + fq;

  const size_t HD = size_t(p.H) * D;
  const int row0 = qt * QT + wave * 32;
  const bool wave_active = row0 < p.P;
  const int qrow = row0 + l32;
  const bool row_ok = qrow < p.P;
  const size_t qbase = ((size_t(b) * p.T + fq) * p.P + qrow) * HD + size_t(h) * D;

  // Q block as the B operand of S^T = K Q^T: lane holds Q[query l32][ks*16 + hl*8 + 0..7]
  bf16x8 qv[8];
  {
    const bf16* q = static_cast<const bf16*>(p.q);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (row_ok) {
        uint4 u = *reinterpret_cast<const uint4*>(q + qbase + ks * 16 + hl * 8);
        qv[ks] = *reinterpret_cast<bf16x8*>(&u);
      } else {
        uint4 z = make_uint4(0, 0, 0, 0);
        qv[ks] = *reinterpret_cast<bf16x8*>(&z);
      }
    }
  }

  const float c = p.scale_log2;
  const int nswa = swa_count(f, p.W);
  const int ndswa = dswa_count(f, p.dil, p.taps);
  Stage st;

  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    const int ntiles = int((nk + KT - 1) / KT);
    float m = -INFINITY;   // running max of the scaled (log2-domain) scores
    float lsum = 0.f;      // running sum over this half-wave's keys
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    __syncthreads();   // the previous branch's last tile is no longer read
    if (ntiles > 0) {
      load_tile(st, p, b, h, branch, f, nswa, nframes, nk, 0, tid);
      store_tile(sm, 0, st, tid);
    }
    for (int t = 0; t < ntiles; ++t) {
      const int buf = t & 1;
      __syncthreads();
      const bool more = t + 1 < ntiles;
      if (more) load_tile(st, p, b, h, branch, f, nswa, nframes, nk, (long long)(t + 1) * KT, tid);

      if (wave_active) {
        // S^T for 64 keys: two 32x32 blocks (keys kb*32 .. +31) x 32 queries
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sm.K[buf][kb * 32 + l32][ks * 16 + hl * 8]);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qv[ks], s[kb], 0, 0, 0);
          }
        }
        // mask keys past the end (last tile only); value r of block kb is key
        // kb*32 + (r/4)*8 + 4*hl + r%4 of the tile
        const long long kleft = nk - (long long)t * KT;
        if (kleft < KT) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb * 32 + (r >> 2) * 8 + 4 * hl + (r & 3);
              if (key >= kleft) s[kb][r] = -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float mnew = fmaxf(m, mt * c);
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        // P^T in bf16, directly in B-operand layout: MFMA (kb, m2) takes values r = m2*8 + 0..7
        bf16x8 pv[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mnew));
            lsum += e;
            pv[kb][r >> 3][r & 7] = static_cast<bf16>(e);
          }
        // O^T += V^T P^T: A operand lane = d row (db*32 + l32), keys of slot i:
        // kb*32 + 16*m2 + 8*(i/4) + 4*hl + i%4
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
              const bf16* vrow = &sm.Vt[buf][db * 32 + l32][kb * 32 + 16 * m2 + 4 * hl];
              const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
              const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
              const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pv[kb][m2], acc[db], 0, 0, 0);
            }
      }
      if (more) store_tile(sm, buf ^ 1, st, tid);
    }

    // ---- epilogue of this branch: normalise, store, keep for the mix ----
    if (wave_active) {
      const float ltot = lsum + __shfl_xor(lsum, 32);
      const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
      Tout* out = static_cast<Tout*>(branch == 0 ? p.o_swa : p.o_dswa);
      const Tout* out_swa = static_cast<const Tout*>(p.o_swa);
      const Tout* og = static_cast<const Tout*>(p.o_gdn);
      Tout* om = static_cast<Tout*>(p.o_mix);
      const float w0 = p.mix_w[h * 3 + 0], w1 = p.mix_w[h * 3 + 1], w2 = p.mix_w[h * 3 + 2];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dcol = db * 32 + j * 8 + 4 * hl;   // 4 consecutive d values r = 4j .. 4j+3
          float o4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = stored_value<Tout>(acc[db][4 * j + e] * inv);
          if (!row_ok) continue;
          store4(out + qbase + dcol, o4);
          if (branch == 1) {
            // the mix reads back this lane's own SWA store and the GDN output
            float s4[4], g4[4], m4[4];
            load4(out_swa + qbase + dcol, s4);
            load4(og + qbase + dcol, g4);
#pragma unroll
            for (int e = 0; e < 4; ++e) m4[e] = w0 * s4[e] + w1 * o4[e] + w2 * g4[e];
            store4(om + qbase + dcol, m4);
          }
        }
    }
  }
}

template <typename Tout>
hipError_t launch_t(const AttnParams& p, hipStream_t st) {
  const long long nqt = (p.P + QT - 1) / QT;
  const long long total = (long long)p.B * p.H * p.T * nqt;
  const long long grid = (total + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_mfma_kernel<Tout>), dim3(unsigned(grid)), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, int out_dt, hipStream_t st) {
  return out_dt == HLTA_BF16 ? launch_t<bf16>(p, st) : launch_t<float>(p, st);
}

}  // namespace hlta
