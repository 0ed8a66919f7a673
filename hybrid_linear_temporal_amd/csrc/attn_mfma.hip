// SWA + DSWA softmax attention with bf16 MFMA on gfx950 (d = 128).
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
//    owns 32 query rows and keeps them in registers as MFMA operands; two
//    workgroups per CU (two waves per SIMD) so one wave's softmax overlaps the
//    other's MFMAs and memory waits;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then holds 32 key scores of one query, which is exactly the
//    B-operand layout of O^T = V^T P^T, so P never goes through LDS;
//  * K and V tiles sit in LDS key-major, 16-byte chunks XOR-permuted per row
//    so that both the K column reads and the transposed V^T reads
//    (ds_read_b64_tr_b16) are free of bank conflicts; tiles go global -> LDS
//    by direct loads (global_load_lds_dwordx4, no staging registers),
//    double-buffered in four separately named LDS objects with one barrier per
//    tile and the next tile in flight during compute;
//  * the key stream of a branch is walked with wave-uniform (frame, token)
//    counters, so tile addresses cost no division;
//  * softmax in the exp2 domain with the scale folded into one FMA; the
//    running max is only raised (and the accumulators rescaled) when a tile's
//    max exceeds it by more than 2^8, which leaves the result unchanged
//    (numerator and denominator share the stale max) and skips most rescales;
//  * workgroups are ordered so each XCD (blockIdx mod 8) walks a contiguous
//    range of (head, frame) items, heaviest frames first, so the query tiles of
//    a frame and the neighbouring frames share K/V tiles in that XCD's L2.
#include "attn_mfma_tiles.h"
#include "hlta_device.h"
#include "hlta_launch.h"

namespace hlta {

namespace {

constexpr int RB = 1;            // 32-row query blocks per wave
constexpr int QT = 4 * 32 * RB;  // query rows per workgroup (128)
constexpr float kLazy = 8.f;     // raise the running max only past this margin (log2 units)

template <typename Tout, bool kRing, bool kLse = false>
__global__ void __launch_bounds__(NT, 2)
attn_mfma_kernel(AttnParams p) {
  // The two buffers are four separate LDS objects addressed only by name (the
  // tile loop is unrolled by two): the compiler then knows that reading the
  // current tile does not touch the buffer the direct loads are filling, and
  // does not wait for them, and every LDS read address is a base register
  // plus an immediate.
  __shared__ Tile sK0, sV0, sK1, sV1;
  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63, hl = lane >> 5, l32 = lane & 31, l16 = lane & 15;

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
  if (skipped(p.ro.skip, b)) return;
  const long long f0b = call_frame(p, b);
  const long long f = f0b + fq;

  const size_t HD = size_t(p.H) * D;
  const int wrow0 = qt * QT + wave * 32 * RB;   // first query row (in the frame) of this wave
  const bool wave_active = wrow0 < p.P;
  const size_t fbase = ((size_t(b) * p.T + fq) * p.P) * HD + size_t(h) * D;

  // Q blocks as B operands of S^T = K Q^T: lane holds Q[row l32 of block rb][ks*16 + hl*8 + 0..7]
  bf16x8 qv[RB][8];
  {
    const bf16* q = static_cast<const bf16*>(p.q);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int qrow = wrow0 + rb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (qrow < p.P) u = *reinterpret_cast<const uint4*>(q + fbase + size_t(qrow) * HD + ks * 16 + hl * 8);
        qv[rb][ks] = *reinterpret_cast<bf16x8*>(&u);
      }
    }
  }

  // direct-load lane offsets of a tile inside one frame: row 16w + 4j + lane/16,
  // source chunk swz(row, lane%16)
  const size_t ts = HD;   // token stride (elements)
  unsigned off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 16 * wave + 4 * j + (lane >> 4);
    off[j] = unsigned(row) * unsigned(ts * sizeof(bf16)) + unsigned(swz(row, lane & 15)) * 16u;
  }
  KeyStream<kRing> kst;
  kst.fstride = size_t(p.P) * HD;
  kst.f0 = f0b;
  kst.R = p.R;
  kst.P = p.P;
  if constexpr (!kRing) {
    const size_t o = size_t(b) * p.T * kst.fstride + size_t(h) * D;
    kst.kmain = uni(static_cast<const bf16*>(p.k) + o);
    kst.vmain = uni(static_cast<const bf16*>(p.v) + o);
    kst.kring = kst.kmain;
    kst.vring = kst.vmain;
  } else {
    const size_t o = size_t(b) * kst.fstride + size_t(h) * D;
    const size_t orr = size_t(b) * p.R * kst.fstride + size_t(h) * D;
    kst.kmain = uni(static_cast<const bf16*>(p.k) + o);
    kst.vmain = uni(static_cast<const bf16*>(p.v) + o);
    kst.kring = uni(static_cast<const bf16*>(p.ring_k) + orr);
    kst.vring = uni(static_cast<const bf16*>(p.ring_v) + orr);
  }

  const float c = p.scale_log2;
  const int nswa = swa_count(f, p.W);
  const int ndswa = dswa_count(f, p.dil, p.taps);
  for (int branch = 0; branch < 2; ++branch) {
    const int nframes = branch == 0 ? nswa : ndswa;
    const long long nk = (long long)nframes * p.P;
    const int ntiles = int((nk + KT - 1) / KT);
    float m[RB], lsum[RB];
    f32x16 acc[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      m[rb] = -INFINITY;
      lsum[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[rb][db][r] = 0.f;
    }

    KeyStream<kRing> ks = kst;
    ks.start(branch == 0 ? f - nswa + 1 : f - p.dil, branch == 0 ? 1 : -p.dil, nframes);
    __syncthreads();   // the previous branch's last tile is no longer read
    auto kleft_of = [&](int t) {
      const long long left = nk - (long long)t * KT;
      return int(left < KT ? (left > 0 ? left : 0) : KT);
    };
    if (ntiles > 0) issue_tile(sK0, sV0, ks, kleft_of(0), off, ts, wave, lane);
    // one tile: Kt/Vt hold tile t, Kn/Vn receive tile t + 1
    auto tile = [&](int t, const Tile& Kt, const Tile& Vt, Tile& Kn, Tile& Vn) __attribute__((always_inline)) {
      wait_vmem();
      __syncthreads();   // tile t is in LDS; nobody reads Kn/Vn any more
      if (t + 1 < ntiles) {
        ks.advance();
        issue_tile(Kn, Vn, ks, kleft_of(t + 1), off, ts, wave, lane);
      }

      if (wave_active) {
        // the compiler's MFMA / LDS-read interleaving strategy: it spreads the
        // V^T operand reads one or two per product through the QK^T products
        // and starts the P V products of the first key block among the
        // exponentials of the second (4.97 -> 4.81 ms per 480P launch against
        // the hand-placed phases alone, same results bit for bit)
        __builtin_amdgcn_iglp_opt(0);
        // S^T: for each key block kb (32 keys) and query block rb
        f32x16 s[RB][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[rb][kb][r] = 0.f;
        // all 16 K operands are read before the first product so the reads
        // pipeline (one at a time, each would wait out the LDS latency)
        bf16x8 ka[8][2];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) ka[ks][kb] = ld_chunk(Kt, kb, l32, 2 * ks + hl);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              s[rb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][kb], qv[rb][ks], s[rb][kb], 0, 0, 0);
          }
        }

        // V^T operands, read now so the softmax below hides their latency
        bf16x8 va[4][2][2];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) va[db][kb][m2] = ld_vt(Vt, kb, m2, hl, db * 32 + (l32 & 16), l16);
        __builtin_amdgcn_sched_barrier(0);
        // mask keys past the end (last tile only); value r of block kb is key
        // kb*32 + (r/4)*8 + 4*hl + r%4 of the tile
        // keys of this tile (uniform: a scalar branch, not an exec mask)
        const int kleft = uni(kleft_of(t));
        if (kleft < KT) {
          // compare the lane-independent part of the key index with kleft - 4*hl
          // (one register, instead of 32 hoisted key indices)
          const int kthr = kleft - 4 * hl;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (kb * 32 + (r >> 2) * 8 + (r & 3) >= kthr) s[rb][kb][r] = -INFINITY;
        }
        bf16x8 pv[RB][2][2];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float mt = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[rb][kb][r]);
          mt = max_xor32(mt) * c;
          // lazy rescale: only when some lane's tile max passes its running max by kLazy
          const bool raise = mt > m[rb] + kLazy;
          if (__ballot(raise) != 0) {
            const float mnew = raise ? fmaxf(m[rb], mt) : m[rb];
            const float alpha = __builtin_amdgcn_exp2f(m[rb] - mnew);
            m[rb] = mnew;
            lsum[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[rb][db][r] *= alpha;
          }
          const float mm = m[rb];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float e = __builtin_amdgcn_exp2f(fmaf(s[rb][kb][r], c, -mm));
              lsum[rb] += e;
              pv[rb][kb][r >> 3][r & 7] = static_cast<bf16>(e);
            }
        }
        // O^T += V^T P^T: A operand lane = d row db*32 + l32, keys of slot i:
        // kb*32 + 16*m2 + 8*(i/4) + 4*hl + i%4
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
                acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][kb][m2], pv[rb][kb][m2], acc[rb][db], 0, 0, 0);
            }
      }
    };
    for (int t = 0; t < ntiles; t += 2) {
      tile(t, sK0, sV0, sK1, sV1);
      if (t + 1 < ntiles) tile(t + 1, sK1, sV1, sK0, sV0);
    }

    // ---- epilogue of this branch: normalise, store ----
    if (wave_active) {
      Tout* out = static_cast<Tout*>(branch == 0 ? p.o_swa : p.o_dswa);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int qrow = wrow0 + rb * 32 + l32;
        const float ltot = sum_xor32(lsum[rb]);
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        if (kLse && hl == 0 && qrow < p.P)
          p.lse[((size_t(branch) * p.B + b) * p.H + h) * (size_t(p.T) * p.P) + size_t(fq) * p.P + qrow] =
              ntiles > 0 ? m[rb] + log2f(ltot) : 0.f;
        if (qrow < p.P) {
          const size_t qbase = fbase + size_t(qrow) * HD;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              float o4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) o4[e] = acc[rb][db][4 * j + e] * inv;
              store4(out + qbase + db * 32 + j * 8 + 4 * hl, o4);   // 4 consecutive d values r = 4j .. 4j+3
            }
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
  if (p.R == 0 && p.lse)   // whole clip, softmax statistics wanted (a separate instantiation)
    hipLaunchKernelGGL((attn_mfma_kernel<Tout, false, true>), dim3(unsigned(grid)), dim3(NT), 0, st, p);
  else if (p.R == 0)
    hipLaunchKernelGGL((attn_mfma_kernel<Tout, false>), dim3(unsigned(grid)), dim3(NT), 0, st, p);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<Tout, true>), dim3(unsigned(grid)), dim3(NT), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams& p, int out_dt, hipStream_t st) {
  return out_dt == HLTA_BF16 ? launch_t<bf16>(p, st) : launch_t<float>(p, st);
}

}  // namespace hlta
