// Kernel launchers of the HLTA library (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/hlta.h"
#include "hlta_device.h"

namespace hlta {

// SWA + DSWA, fp32 arithmetic, any supported d and dtype.
hipError_t launch_attn_generic(const AttnParams& p, int d, int in_dt, int out_dt, hipStream_t st);
// SWA + DSWA with bf16 MFMA (bf16 inputs, d = 128).
hipError_t launch_attn_mfma(const AttnParams& p, int out_dt, hipStream_t st);
// o_mix = per-head weighted sum of the three stored branch outputs
// ([ntok, H, d] each, out dtype), d a multiple of 8; rows of rollouts in
// skip (rollout_tokens tokens each) are not written.
hipError_t launch_mix(const void* o_swa, const void* o_dswa, const void* o_gdn, void* o_mix, const float* mix_w,
                      long long ntok, int H, int d, int out_dt, hipStream_t st, unsigned long long skip = 0,
                      long long rollout_tokens = 1);

// FP8 variant of the softmax branches: SWA + DSWA on e4m3 codes (q, k, v of p)
// with float32 scales [B, H, 3] (q, k, v per head), d = 128, P >= 64.
hipError_t launch_attn_fp8(const AttnParams& p, const float* scales, int out_dt, hipStream_t st);
// e4m3 codes of q, k, v [B, L, H, d] (dt) with per-(b, h, tensor) scales.
hipError_t launch_quantize_e4m3(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
                                float* scales, int B, long long L, int H, int d, int dt, hipStream_t st);

// Gated delta rule, chunked form, fp32 arithmetic (any supported d, C, dtype).
hipError_t launch_gdn_generic(const GdnParams& p, int d, int C, int in_dt, int out_dt, hipStream_t st);
// Gated delta rule, chunked form with bf16 MFMA (bf16 inputs, d = 128, C = 64),
// G segments of seg_chunks chunks per (batch row, head) run side by side;
// workspace: gdn_seg_record_bytes(B, H, n_chunks) + gdn_seg_map_bytes(B, H, G, 128) bytes.
hipError_t launch_gdn_seg(const GdnParams& p, int G, int seg_chunks, void* workspace, int out_dt, hipStream_t st);

// dst = src (src non-null) or dst = 0, bytes a multiple of 4; one kernel launch.
hipError_t launch_copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t st);

// Measured ceilings: a dense bf16 MFMA loop (workgroups x 4 waves, iters x 8
// MFMA 32x32x16 per wave) and a 16-byte streaming copy of bytes (multiple of 16).
hipError_t launch_ceiling_mfma(float* sink, unsigned long long* clocks, int workgroups, int iters, hipStream_t st);
hipError_t launch_ceiling_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

// Copy n_frames latent frames [B, frames, P, H, d] from src (frames src_f0..)
// into ring slots (frame g -> slot g mod R). elem = element bytes.
hipError_t launch_ring_store(const void* src, long long src_frames, long long src_f0, void* ring,
                             int R, long long first_frame, long long n_frames, int B, long long frame_elems,
                             int elem, hipStream_t st);

// Rotary embedding of the softmax branches (reading in rope.hip): q, k
// [B, L, H, d] (dt) -> rotated copies qr, kr; token t of row b sits in frame
// (per_rollout ? ro.frame[b] : f0) + t / P; rollouts in ro.skip are left alone.
hipError_t launch_rope_qk(const void* q, const void* k, void* qr, void* kr, int B, long long L, int H, int d, int P,
                          int grid_w, float theta, int dt, long long f0, int per_rollout, const RolloutFrames& ro,
                          hipStream_t st);
// The same in place over the ring slots of frames first .. first+n-1.
hipError_t launch_rope_ring(void* ring, int B, int R, long long first, int n, int H, int d, int P, int grid_w,
                            float theta, int dt, hipStream_t st);

// Streaming with a position per rollout: src [B, P, H, d] holds one frame per
// rollout; rollout b's goes to ring slot sel.frame[b] mod R (rollouts in
// sel.skip are left alone).
hipError_t launch_ring_store_rollouts(const void* src, void* ring, int R, int B, long long frame_elems, int elem,
                                      const RolloutFrames& sel, hipStream_t st);

// Softmax-branch backward with bf16 MFMA (bf16 q, k, v, d_mix and stored
// outputs, d = 128, P >= 64): lse and dsum are [2, B, H, L] fp32 scratch
// (lse given: filled by the forward already, not recomputed); dq, dk, dv
// [B, L, H, d] fp32 are written (not accumulated).
hipError_t launch_attn_bwd_mfma(const AttnParams& p, const void* d_mix, const void* o_swa, const void* o_dswa,
                                const float* mix_w, float* lse, bool lse_given, float* dsum, float* dq, float* dk,
                                float* dv, float scale, hipStream_t st);

// Backward of the operator (bwd.hip): fp32 gradients of q, k, v [B, L, H, d],
// a, b [B, L, H], mix_w [H, 3] and S0 [B, H, d, d] given d_mix (out dtype).
// attn and gdn describe the forward (attn.scale_log2 set; gdn.n_chunks =
// ceil(L / C)); the stored forward outputs feed the mix-weight gradient.
struct BwdArgs {
  AttnParams attn;
  GdnParams gdn;
  const void* d_mix;
  const float* mix_w;
  const void* o_swa;
  const void* o_dswa;
  const void* o_gdn;
  float* dq;
  float* dk;
  float* dv;
  float* da;
  float* db;
  float* dmix_w;
  float* dS0;        // or null
  float* lse2;       // [2, B*L*H] workspace: softmax row statistics
  float* dsum;       // [2, B*L*H] workspace
  float* Am;         // [B*H, n_chunks, d, d] workspace: per-chunk transition of the memory
  float* Um;         //   ... the chunk's own state from zero
  float* Xm;         //   ... the chunk's own adjoint from zero
  float* Sst;        //   ... state at the chunk's start
  float* Rin;        //   ... adjoint reaching the chunk's end
  float* slots;      // [n_slots, slot_floats] workspace: one slot per chunk of the memory's backward
  int n_slots;
  size_t slot_floats;
  float* dw_part;    // [H, dw_slices, 3] workspace
  int dw_slices;
  int C;
  float scale;
  int attn_mfma;     // softmax branches on the bf16 MFMA kernels (bf16 in and out, d = 128, P >= 64)
  int lse_given;     // lse2 holds the forward's statistics (MFMA path only)
};

// The gated delta rule's backward in matrix form (per chunk): phase 0 the
// chunk maps Am, Um, Xm; phase 2 the two chains over chunks (Sst, Rin,
// dS0); phase 1 (after the chains) the token gradients.
hipError_t launch_gdn_bwd_mat(const BwdArgs& x, int d, int in_dt, int out_dt, int phase, hipStream_t st);
hipError_t launch_bwd(const BwdArgs& x, int d, int in_dt, int out_dt, hipStream_t st);

}  // namespace hlta
