// SWA + DSWA softmax attention on e4m3 inputs with the gfx950 scaled 8-bit
// MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), d = 128: the FP8 variant of the
// softmax branches. The pages mention low-precision attention without a
// method; the reading implemented: q, k, v arrive as e4m3 codes with one
// float32 scale per (batch row, head, tensor) (fp8_ops.hip makes them), the
// products accumulate in fp32, the softmax runs in fp32 exactly as in the
// bf16 kernel, and P is rounded to e4m3 for the P V product. The result is
// exact attention over the dequantised inputs up to the rounding of P.
//
// Same structure as the bf16 kernel (attn_mfma.hip): 4 waves x 32 query rows
// per workgroup, S^T = K Q^T so a lane's 32 scores are already the B operand
// of O^T = V^T P^T, 64-key K and V tiles loaded global -> LDS by direct loads,
// double-buffered, lazy rescale of the running max. What changes with 8-bit
// operands:
//  * one MFMA covers 64 of the reduction index: QK^T is 2 x 2 MFMAs per tile
//    (two 32-key blocks, two 64-wide halves of d), P V is 4 (one per 32-row d
//    block) plus one with an all-ones A operand, whose output is the sum of the
//    rounded P of each query: numerator and denominator see the same P;
//  * MFMA operand layout (checked on the GPU with a probe): lane l holds row
//    l%32 and the 32 reduction indices 32(l/32) .. 32(l/32)+31 of A and B
//    alike, so any permutation of the reduction index shared by A and B gives
//    the same product. A lane's scores are keys kb*32 + 8(r/4) + 4(l/32) + r%4;
//    byte j = 16 kb + r of its P operand is that key, and the V^T operand is
//    read in the same key order;
//  * tiles are 64 rows of 128 bytes; 16-byte chunk c of row r sits at chunk
//    position c ^ ((r/2) mod 8), which spreads both the K operand reads
//    (ds_read_b128, 16 rows per pass) and the transposed V^T reads over all
//    banks;
//  * V^T comes from ds_read_b64_tr_b8: within 16 lanes, lane u receives as
//    byte t byte u%8 of the 8 bytes addressed by lane 2t + u/8 (probed), so
//    lane v of a 16-lane group addresses the key of byte t = v/2 and the
//    columns 8(v%2) .. of its group's 16-column block.
#include "attn_mfma_tiles.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef unsigned char u8;

constexpr int QT = 128;          // query rows per workgroup: 4 waves x 32
constexpr float kLazy = 8.f;     // raise the running max only past this margin (log2 units); P <= 2^8 < 448
constexpr int kScaleOne = 127;   // E8M0 block scale 2^0 of the MFMA

__device__ __forceinline__ f32x16 mfma8(const v8i& a, const v8i& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kScaleOne, 0, kScaleOne);
}

template <typename Tout>
__global__ void __launch_bounds__(NT, 2)
attn_fp8_kernel(AttnParams p, const float* scales) {
  __shared__ Tile8 sK0, sV0, sK1, sV1;
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, g = lane >> 5, l32 = lane & 31;

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

  const size_t HD = size_t(p.H) * D;   // token stride, bytes of codes and elements of outputs
  const int wrow0 = qt * QT + wave * 32;
  const bool wave_active = wrow0 < p.P;
  const size_t fbase = ((size_t(b) * p.T + fq) * p.P) * HD + size_t(h) * D;
  const float sq = scales[size_t(bh) * 3], sk = scales[size_t(bh) * 3 + 1], sv = scales[size_t(bh) * 3 + 2];
  const float c = p.scale_log2 * sq * sk;

  // Q operand (B of S^T = K Q^T): lane holds q codes of row l32, columns 64 ks + 32 g .. +31
  v8i qv[2];
  {
    const u8* q = static_cast<const u8*>(p.q);
    const int qrow = wrow0 + l32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
      if (qrow < p.P) {
        const uint4* src = reinterpret_cast<const uint4*>(q + fbase + size_t(qrow) * HD + 64 * ks + 32 * g);
        lo = src[0];
        hi = src[1];
      }
      qv[ks] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
  }
  // all-ones A operand (e4m3 1.0 = 0x38): its product with P is the column sum of P
  const int one4 = 0x38383838;
  const v8i ones = {one4, one4, one4, one4, one4, one4, one4, one4};

  // direct-load lane offsets: row 16w + 8j + lane/8, source chunk swz8(row, lane%8)
  const size_t ts = HD;
  unsigned off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 16 * wave + 8 * j + (lane >> 3);
    off[j] = unsigned(row) * unsigned(ts) + unsigned(swz8(row, lane & 7)) * 16u;
  }
  // K operand addresses: row kb*32 + l32, logical chunks 4ks + 2g + e (kb adds 4096 bytes)
  int koff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 2; ++e) koff[ks][e] = l32 * 128 + swz8(l32, 4 * ks + 2 * g + e) * 16;
  // V^T addresses: lane v of its 16-lane group reads key 16 q + R (q = 0..3 adds 2048
  // bytes), R = 8 (t/4) + 4 g + t%4 with t = v/2, columns 32 db + 16 G' + 8 (v%2)
  int voff[4];
  {
    const int v = lane & 15, t = v >> 1, gp = (lane >> 4) & 1;
    const int R = 8 * (t >> 2) + 4 * g + (t & 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) voff[db] = R * 128 + swz8(R, 2 * db + gp) * 16 + 8 * (v & 1);
  }

  KeyStream<false, u8> kst;
  kst.fstride = size_t(p.P) * HD;
  kst.P = p.P;
  {
    const size_t o = size_t(b) * p.T * kst.fstride + size_t(h) * D;
    kst.kmain = uni(static_cast<const u8*>(p.k) + o);
    kst.vmain = uni(static_cast<const u8*>(p.v) + o);
  }

  const int nswa = swa_count(f, p.W);
  const int ndswa = dswa_count(f, p.dil, p.taps);
  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    const int ntiles = int((nk + KT - 1) / KT);
    float m = -INFINITY;
    f32x16 acc[4], accs;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      accs[r] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db][r] = 0.f;
    }

    KeyStream<false, u8> ks = kst;
    ks.start(branch == 0 ? f - nswa + 1 : f - p.dil, branch == 0 ? 1 : -p.dil, nframes);
    __syncthreads();   // the previous branch's last tile is no longer read
    auto kleft_of = [&](int t) {
      const long long left = nk - (long long)t * KT;
      return int(left < KT ? (left > 0 ? left : 0) : KT);
    };
    if (ntiles > 0) issue_tile(sK0, sV0, ks, kleft_of(0), off, ts, wave, lane);
    auto tile = [&](int t, const Tile8& Kt, const Tile8& Vt, Tile8& Kn, Tile8& Vn) __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();   // tile t is in LDS; nobody reads Kn/Vn any more
      if (t + 1 < ntiles) {
        ks.advance();
        issue_tile(Kn, Vn, ks, kleft_of(t + 1), off, ts, wave, lane);
      }
      if (!wave_active) return;
      // K operands (both key blocks, both halves of d), read before the products
      v8i ka[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const uint4 lo = *reinterpret_cast<const uint4*>(at(Kt, koff[k2][0], kb * 4096));
          const uint4 hi = *reinterpret_cast<const uint4*>(at(Kt, koff[k2][1], kb * 4096));
          ka[kb][k2] = v8i{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 z;
#pragma unroll
        for (int r = 0; r < 16; ++r) z[r] = 0.f;
        s[kb] = mfma8(ka[kb][0], qv[0], z);
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma8(ka[kb][1], qv[1], s[kb]);
      // V^T operands, read now so the softmax hides their latency
      v8i va[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        v2i x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          x[q] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(at(Vt, voff[db], q * 2048)));
        va[db] = v8i{x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
      }
      __builtin_amdgcn_sched_barrier(0);
      // mask keys past the end (last tile only): value r of block kb is key
      // kb*32 + (r/4)*8 + 4g + r%4 of the tile
      const int kleft = uni(kleft_of(t));
      if (kleft < KT) {
        const int kthr = kleft - 4 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + (r >> 2) * 8 + (r & 3) >= kthr) s[kb][r] = -INFINITY;
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = max_xor32(mt) * c;
      const bool raise = mt > m + kLazy;
      if (__ballot(raise) != 0) {
        const float mnew = raise ? fmaxf(m, mt) : m;
        const float alpha = __builtin_amdgcn_exp2f(m - mnew);
        m = mnew;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          accs[r] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db) acc[db][r] *= alpha;
        }
      }
      // P in e4m3, byte j = 16 kb + r of the B operand
      v8i pv;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = w >> 2, r0 = (w & 3) * 4;
        float e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + u], c, -m));
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
        pv[w] = word;
      }
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = mfma8(va[db], pv, acc[db]);
      accs = mfma8(ones, pv, accs);
    };
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, sK0, sV0, sK1, sV1);
      if (t + 1 < ntiles) tile(t + 1, sK1, sV1, sK0, sV0);
    }

    // ---- epilogue: normalise by the sum of the rounded P, dequantise v, store ----
    if (wave_active) {
      Tout* out = static_cast<Tout*>(branch == 0 ? p.o_swa : p.o_dswa);
      const int qrow = wrow0 + l32;
      const float ltot = accs[0];
      const float inv = ltot > 0.f ? sv / ltot : 0.f;
      if (qrow < p.P) {
        const size_t qbase = fbase + size_t(qrow) * HD;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float o4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = acc[db][4 * j + e] * inv;
            store4(out + qbase + db * 32 + j * 8 + 4 * g, o4);
          }
      }
    }
  }
}

template <typename Tout>
hipError_t launch_t(const AttnParams& p, const float* scales, hipStream_t st) {
  const long long nqt = (p.P + QT - 1) / QT;
  const long long total = (long long)p.B * p.H * p.T * nqt;
  const long long grid = (total + kXcds - 1) / kXcds * kXcds;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fp8_kernel<Tout>), dim3(unsigned(grid)), dim3(NT), 0, st, p, scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fp8(const AttnParams& p, const float* scales, int out_dt, hipStream_t st) {
  return out_dt == HLTA_BF16 ? launch_t<bf16>(p, scales, st) : launch_t<float>(p, scales, st);
}

}  // namespace hlta
