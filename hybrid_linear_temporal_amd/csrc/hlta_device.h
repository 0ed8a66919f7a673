// Device-side helpers and kernel parameter blocks of the HLTA library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace hlta {

using bf16 = __bf16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// round-to-nearest-even (gfx950 converts with v_cvt_pk_bf16_f32)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Value of x after a round trip through T (what a store of x leaves in memory).
template <typename T> __device__ __forceinline__ float stored_value(float x) {
  return to_f32(from_f32<T>(x));
}

// Parameters of the softmax branches (SWA + DSWA).
// Full mode (R == 0): queries and keys come from q, k, v of T frames.
// Stream mode (R > 0): the call's single query frame is absolute frame f0;
// its own K/V come from k, v; earlier frames g from ring slot g mod R.
// Rollouts left out of a launch have their bit set in a skip mask: their
// workgroups return at once, so nothing of theirs is read or written.
constexpr int kMaxRollouts = 64;
__device__ __forceinline__ bool skipped(unsigned long long skip, int b) {
  return b < kMaxRollouts && ((skip >> b) & 1ull) != 0;
}

// Frame index per rollout and the rollouts left out (kernel argument).
struct RolloutFrames {
  unsigned long long skip;
  long long frame[kMaxRollouts];
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  const void* ring_k;
  const void* ring_v;
  void* o_swa;
  void* o_dswa;
  int B, H, T, P;        // T = query frames of this call
  int W, dil, taps;
  int R;                 // ring frames (stream mode) or 0
  long long f0;          // absolute index of query frame 0
  float scale_log2;      // softmax scale * log2(e)
  // Streaming with a position per rollout (T = 1): rollout b's query frame is
  // ro.frame[b]; rollouts in ro.skip are left out entirely (also without it).
  int per_rollout;
  RolloutFrames ro;
  // Optional (whole-clip calls): per query row and branch, the log2 of the
  // softmax denominator with scores in log2 units, [2, B, H, T*P]; 0 for a
  // row with no keys.
  float* lse;
};

// Absolute index of the call's first query frame for rollout b.
__device__ __forceinline__ long long call_frame(const AttnParams& p, int b) {
  return p.per_rollout ? p.ro.frame[b] : p.f0;
}

// Key frame g (absolute index) of batch row b, head h: pointer to its token 0.
// Tokens of a frame are H*D elements apart.
template <typename T, int D>
__device__ __forceinline__ const T* key_frame_ptr(const T* main, const T* ring, const AttnParams& p,
                                                  int b, int h, long long g) {
  if (p.R == 0)
    return main + ((size_t(b) * p.T * p.P + size_t(g) * p.P) * p.H + h) * D;
  if (g == call_frame(p, b))
    return main + (size_t(b) * p.P * p.H + h) * D;
  const int slot = int(g % p.R);
  return ring + ((size_t(b) * p.R + slot) * p.P * p.H + h) * D;
}

// Decay and write gates of one token as the memory uses them: log a (floored)
// and b, from the given gates or, with logits, from log sigmoid(x_a) and
// sigmoid(x_b); log sigmoid(x) = min(x, 0) - log1p(exp(-|x|)) has no
// cancellation for either sign.
__device__ __forceinline__ void gate_values(float xa, float xb, int logits, float floor_log_a, float& la,
                                            float& bi) {
  if (logits) {
    la = fmaxf(fminf(xa, 0.f) - log1pf(expf(-fabsf(xa))), floor_log_a);
    bi = 1.f / (1.f + expf(-xb));
  } else {
    la = fmaxf(logf(xa), floor_log_a);
    bi = xb;
  }
}
__device__ __forceinline__ void load_gates(const float* a, const float* b, size_t i, int logits, float floor_log_a,
                                           float& la, float& bi) {
  gate_values(a[i], b[i], logits, floor_log_a, la, bi);
}

// Frame sets of query frame f (absolute): SWA reads frames f-nswa+1 .. f,
// DSWA reads f - dil*(s+1) for s < ndswa.
__device__ __forceinline__ int swa_count(long long f, int W) {
  return int(f + 1 < W ? f + 1 : W);
}
__device__ __forceinline__ int dswa_count(long long f, int dil, int taps) {
  const long long n = f / dil;
  return int(n < taps ? n : taps);
}
__device__ __forceinline__ long long branch_frame(int branch, long long f, int nswa, int dil, int s) {
  return branch == 0 ? f - nswa + 1 + s : f - (long long)dil * (s + 1);
}

// Parameters of the gated delta rule kernels.
struct GdnParams {
  const void* q;
  const void* k;
  const void* v;
  const float* a;
  const float* b;
  const float* S0;       // [B, H, D, D] or null
  float* S_out;          // [B, H, D, D] or null (may alias S0)
  void* o;               // [B, L, H, D]
  unsigned char* ws;     // per-chunk records
  size_t rec_bytes;
  int B, H;
  long long L;
  int n_chunks;
  int l2norm;
  int gate_logits;           // a, b hold logits: the gates are sigmoid(a), sigmoid(b)
  unsigned long long skip;   // rollouts left out (bit b)
};

}  // namespace hlta
