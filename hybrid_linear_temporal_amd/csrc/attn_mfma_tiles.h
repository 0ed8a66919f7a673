// Tile machinery shared by the MFMA softmax-branch kernels (bf16 forward and
// backward, e4m3 forward; d = 128): 64-row tiles in LDS (256-byte rows of
// bf16, 128-byte rows of e4m3) with a per-row XOR permutation of the 16-byte
// chunks, direct global -> LDS loads, the walk over the rows of a branch's
// frames as one virtual sequence, and the bf16 MFMA operand reads (row chunks
// and transposed reads) of gfx950.
#pragma once

#include "hlta_device.h"

namespace hlta {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int D = 128;           // head dim
constexpr int KT = 64;           // keys per tile
constexpr int NT = 256;          // threads
constexpr int kXcds = 8;

// one K or V tile: 64 rows of kRowBytes, 16-byte chunks permuted per row
template <int kRowBytes>
struct TileOf {
  uint4 row[KT][kRowBytes / 16];
};
using Tile = TileOf<256>;    // bf16 rows (swz)
using Tile8 = TileOf<128>;   // e4m3 rows (swz8)

// 16-byte chunk c of key row r sits at chunk position c ^ f(r mod 16), with f
// swapping the two 2-bit halves of the row index. A 256-byte row spans all 64
// LDS banks, so only the position matters: f is a bijection, so the 16 rows of
// a K column read land on 16 positions, and the 8 rows x 4 chunks of a
// transposed V read (rows 4*hl + e) reach all 16 positions twice, the minimum
// two passes. With the plain c ^ (r mod 16) those V reads hit 8 positions
// only (four-way bank conflicts, measured at 2.8x the time).
__device__ __forceinline__ int swz(int r, int c) {
  const int x = r & 15;
  return c ^ (((x & 3) << 2) | (x >> 2));
}

// 128-byte rows (8 chunks, half the banks): chunk c of row r at position
// c ^ ((r / 2) mod 8), which spreads both 16-row operand reads (two rows per
// bank set) and the 8-bit transposed reads over all banks.
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int kRowBytes>
__device__ __forceinline__ int swz_row(int r, int c) {
  static_assert(kRowBytes == 256 || kRowBytes == 128, "tile rows are 256 or 128 bytes");
  if constexpr (kRowBytes == 256) return swz(r, c);
  else return swz8(r, c);
}

// Wave-uniform values kept in scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ const T* uni(const T* ptr) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(ptr);
  const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(u));
  const unsigned hi = __builtin_amdgcn_readfirstlane(unsigned(u >> 32));
  return reinterpret_cast<const T*>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Walks the virtual key sequence of one branch tile by tile (the key-major
// backward walks the queries of the frames that read a key frame the same way). A tile of 64
// keys spans at most two frames (P >= 64); all fields are wave-uniform.
// Frames of a branch are g, g + step, ...: step 1 for SWA (oldest first),
// -dil for DSWA. In stream mode the call's own frame f0 comes from the main
// tensors and earlier frames from ring slot g mod R. E is the element type
// (bf16, or unsigned char for e4m3 codes); strides count elements.
template <bool kRing, typename E = bf16>
struct KeyStream {
  const E* kmain;        // token 0 of frame 0 (full mode) or of the call's frame (stream mode), head h
  const E* vmain;
  const E* kring;        // token 0 of ring slot 0, head h (stream mode)
  const E* vring;
  size_t fstride;        // elements between consecutive frames: P*H*D
  long long f0;
  int R;
  long long g;           // current frame
  int step, left, P;     // frame step, frames after the current one, tokens per frame
  int pk;                // current tile starts at token pk of the current frame
  const E* k0;           // token 0 of the current frame
  const E* v0;
  const E* k1;           // token 0 of the next frame (the current one if none)
  const E* v1;

  __device__ __forceinline__ void frame_ptrs(long long gg, const E*& kb, const E*& vb) const {
    if constexpr (!kRing) {
      const size_t off = size_t(gg) * fstride;
      kb = uni(kmain + off);
      vb = uni(vmain + off);
    } else {
      if (gg == f0) {
        kb = kmain;
        vb = vmain;
      } else {
        const size_t off = size_t(unsigned(gg) % unsigned(R)) * fstride;
        kb = uni(kring + off);
        vb = uni(vring + off);
      }
    }
  }
  __device__ __forceinline__ void start(long long g_first, int step_, int nframes) {
    g = g_first;
    step = step_;
    left = nframes - 1;
    pk = 0;
    if (nframes > 0) frame_ptrs(g, k0, v0);
    if (nframes > 1) frame_ptrs(g + step, k1, v1);
    else {
      k1 = k0;
      v1 = v0;
    }
  }
  __device__ __forceinline__ void advance() {
    pk += KT;
    if (pk >= P) {
      pk -= P;
      g += step;
      --left;
      k0 = k1;
      v0 = v1;
      if (left > 0) frame_ptrs(g + step, k1, v1);
    }
  }
};

// Buffer resource over [base, base + bytes): 32-bit lane offsets on a scalar base.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// Direct global -> LDS copy of the current tile: wave w moves rows 16w .. 16w+15,
// 1 KB per instruction (four 256-byte or eight 128-byte rows); lane i lands at
// chunk position i % n of row 16w + (64/n) j + i/n (n chunks per row) and so
// loads the chunk that the swizzle puts there. A tile
// inside one frame (the common case) loads through buffer resources with the
// precomputed lane offsets `off` (kRowBytes / 64 of them, no per-lane
// address arithmetic); a tile
// across a frame boundary or past the end of the sequence computes each lane's
// row, and rows past the end re-read the last valid row (finite data; their
// scores are masked, so they contribute exactly zero).
template <bool kRing, bool kV = true, typename E = bf16, int kRowBytes = 256>
__device__ __forceinline__ void issue_tile(TileOf<kRowBytes>& Kd, TileOf<kRowBytes>& Vd,
                                           const KeyStream<kRing, E>& ks, int kleft,
                                           const unsigned* off, size_t ts, int wave, int lane) {
  constexpr int kChunks = kRowBytes / 16;   // 16-byte chunks per row
  constexpr int kRows = 64 / kChunks;       // rows per instruction
  constexpr int kInst = 16 / kRows;         // instructions per wave
  if (ks.pk + KT <= ks.P && kleft >= KT) {
    const unsigned bytes = unsigned(KT * ts * sizeof(E));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(ks.k0 + size_t(ks.pk) * ts, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(ks.v0 + size_t(ks.pk) * ts, bytes);
#pragma unroll
    for (int j = 0; j < kInst; ++j) {
      const int r0 = 16 * wave + kRows * j;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(&Kd.row[r0][0]), 16,
                                               off[j], 0, 0, 0);
      if constexpr (kV)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(&Vd.row[r0][0]),
                                                 16, off[j], 0, 0, 0);
    }
    return;
  }
  // Rows 0 .. split-1 of the tile lie in the current frame, the rest in the
  // next one: one buffer resource per frame, each lane loading under the
  // exec mask of its frame. (Buffer loads only: with a FLAT-encoded
  // global_load_lds anywhere in the loop the compiler cannot tell LDS reads
  // from those loads in the LDS counter and waits for every outstanding LDS
  // read before the first product that needs one of them.)
  const int split = ks.P - ks.pk;
  const unsigned bytes = unsigned(KT * ts * sizeof(E));
  const __amdgpu_buffer_rsrc_t rka = make_rsrc(ks.k0 + size_t(ks.pk) * ts, bytes);
  const __amdgpu_buffer_rsrc_t rva = make_rsrc(ks.v0 + size_t(ks.pk) * ts, bytes);
  const __amdgpu_buffer_rsrc_t rkb = make_rsrc(ks.k1, bytes);
  const __amdgpu_buffer_rsrc_t rvb = make_rsrc(ks.v1, bytes);
#pragma unroll
  for (int j = 0; j < kInst; ++j) {
    const int r0 = 16 * wave + kRows * j;
    const int row = r0 + lane / kChunks;
    const int rr = row < kleft ? row : kleft - 1;
    const int c = swz_row<kRowBytes>(row, lane % kChunks);
    const bool here = rr < split;
    const unsigned o = unsigned((here ? rr : rr - split) * ts * sizeof(E)) + unsigned(c) * 16u;
    auto* kd = (__attribute__((address_space(3))) void*)(&Kd.row[r0][0]);
    auto* vd = (__attribute__((address_space(3))) void*)(&Vd.row[r0][0]);
    if (here) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rka, kd, 16, o, 0, 0, 0);
      if constexpr (kV) __builtin_amdgcn_raw_ptr_buffer_load_lds(rva, vd, 16, o, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkb, kd, 16, o, 0, 0, 0);
      if constexpr (kV) __builtin_amdgcn_raw_ptr_buffer_load_lds(rvb, vd, 16, o, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }   // vmcnt(0)
// Lanes l and l ^ 32 combined without LDS: v_permlane32_swap on two copies of
// x leaves (x[l], x[l^32]) in lanes below 32 and (x[l^32], x[l]) above (lane
// layout checked on the GPU). The results are copied out of the returned
// vector before the bit casts: casting the vector elements in place reads
// element 0 twice with this compiler.
__device__ __forceinline__ void pair_xor32(float x, float& a, float& b) {
  const unsigned xa = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(xa, xa, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a, b;
  pair_xor32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a, b;
  pair_xor32(x, a, b);
  return a + b;
}

// Address of (lane part + constant part) inside a tile. The lane part is made
// provably less than kLaneBound bytes (a power of two no smaller than the
// largest lane part of the caller), and the constant part is added to the
// tile's own LDS address first, so the compiler can fold both into the
// instruction's 16-bit immediate offset and one set of lane address registers
// serves the buffers and key blocks. (With the lane part added first it kept
// a register per buffer and lane part, and the forward kernel spilled.)
template <int kLaneBound = 0, int kRowBytes>
__device__ __forceinline__ const char* at(const TileOf<kRowBytes>& t, int lane_off, int const_off) {
  constexpr unsigned kMask = (kLaneBound ? unsigned(kLaneBound) : unsigned(sizeof(TileOf<kRowBytes>))) - 1u;
  return (reinterpret_cast<const char*>(&t) + const_off) + (unsigned(lane_off) & kMask);
}

// 8 consecutive d values (chunk c) of key row kb*32 + l32
__device__ __forceinline__ bf16x8 ld_chunk(const Tile& t, int kb, int l32, int c) {
  return *reinterpret_cast<const bf16x8*>(at<32 * 256>(t, l32 * 256 + swz(l32, c) * 16, kb * 32 * 256));
}

// V^T operand of one 32x32x16 MFMA: lane = d row (d0 + l16 inside its 16-lane group),
// slots 0..3 = keys k0 .. k0+3, slots 4..7 = keys k0+8 .. k0+11 with
// k0 = kb*32 + 16*m2 + 4*hl, read transposed: lane 4e+q of the group addresses
// key row k0+e (+8), d columns d0 + 4q .. +3. Rows kb*32 + 16*m2 + x share
// their swizzle with row x, so only x enters the lane part.
__device__ __forceinline__ bf16x8 ld_vt(const Tile& t, int kb, int m2, int hl, int d0, int l16) {
  const int e = l16 >> 2, q = l16 & 3;
  const int dcol = d0 + 4 * q;
  const int x0 = 4 * hl + e, x1 = x0 + 8;
  const int kc = (kb * 32 + 16 * m2) * 256;
  const char* p0 = at<16 * 256>(t, x0 * 256 + swz(x0, dcol >> 3) * 16 + (dcol & 7) * 2, kc);
  const char* p1 = at<16 * 256>(t, x1 * 256 + swz(x1, dcol >> 3) * 16 + (dcol & 7) * 2, kc);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 x = {static_cast<bf16>(v[0]), static_cast<bf16>(v[1]), static_cast<bf16>(v[2]), static_cast<bf16>(v[3])};
  *reinterpret_cast<bf16x4*>(p) = x;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  f32x4 x = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = x;
}

}  // namespace
}  // namespace hlta
