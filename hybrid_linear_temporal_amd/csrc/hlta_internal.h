// Internal host-side declarations shared by the HIP-free host layer
// (hlta_host.cpp) and the launch layer (hlta_api.hip). No HIP types here, so
// the host layer also builds with plain g++ into a CPU test binary.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/hlta.h"

namespace hlta {

// Which kernel family runs each branch.
enum class Impl : int { Generic = 1, Mfma = 2 };

struct Plan {
  Impl attn = Impl::Generic;
  Impl gdn = Impl::Generic;
  int64_t L = 0;            // tokens per batch row in this call
  int64_t n_chunks = 0;     // ceil(L / C)
  size_t ws_gdn = 0;        // bytes of GDN scratch
  size_t ws_rope_off = 0;   // rotated q, then rotated k (rotary embedding on), each ws_rope_bytes
  size_t ws_rope_bytes = 0;
  size_t ws_total = 0;      // bytes the caller must supply
  float scale = 0.f;        // resolved softmax scale
};

// Record a failure message for hlta_last_error() and return the status.
hlta_status fail(hlta_status s, const std::string& msg);
void clear_error();

// Config checks that need no GPU. Returns HLTA_OK or an error (message set).
hlta_status check_config(const hlta_config* cfg);

// Kernel selection and workspace layout for a call over L tokens per row.
hlta_status make_plan(const hlta_config* cfg, int64_t L, Plan* plan);

// Workspace of the backward over L tokens per row, all fp32, 256-byte
// aligned: per-row softmax statistics of both branches (two arrays); six
// d x d matrices per chunk of C = gdn_chunk tokens (transition and its
// transpose, own state, own adjoint, start state, adjoint at the end); the recomputed states of one
// chunk per slot (one slot per workgroup of the token pass); partial sums of
// the mix-weight gradient.
constexpr int kBwdSlots = 512;
constexpr int kDwSlices = 128;
struct BwdPlan {
  size_t stats_bytes = 0;   // each of the two: [2, B*L*H]
  size_t mat_off = 0, mat_bytes = 0;   // each of the six: [B*H*n_chunks, d, d]
  size_t slot_off = 0;
  int n_slots = 0;
  size_t part_off = 0;
  size_t total = 0;
};
hlta_status make_bwd_plan(const hlta_config* cfg, BwdPlan* plan);

// Is there an MFMA kernel for this shape?
bool mfma_attn_supported(const hlta_config* cfg);
bool mfma_gdn_supported(const hlta_config* cfg);

// Per-chunk record sizes of the GDN scratch (in bytes).
size_t gdn_generic_record_bytes(int C, int d);

// Record of one chunk for the MFMA gated-delta-rule kernels (C = 64, d = 128):
//   Wn   bf16 [C][d]  -W = -T diag(b gamma) K^   (row per token)
//   UpT  bf16 [d][C]  U'^T = (T diag(b) V)^T     (row per value channel)
//   Aqk  bf16 [C][C]  exp(g_i - g_j) q^_i.k^_j, j <= i
//   sq   f32  [C]     gamma_i / ||q_i||          (scales rows of Q S^T)
//   sk   f32  [C]     gamma_C / (gamma_i ||k_i||) (scales rows of U in the state update)
//   gC   f32          gamma_C
struct GdnMfmaRec {
  static constexpr size_t C = 64, D = 128;
  static constexpr size_t WN = 0;
  static constexpr size_t UPT = WN + 2 * C * D;
  static constexpr size_t AQK = UPT + 2 * D * C;
  static constexpr size_t SQ = AQK + 2 * C * C;
  static constexpr size_t SK = SQ + 4 * C;
  static constexpr size_t GC = SK + 4 * C;
  static constexpr size_t BYTES = (GC + 16 + 255) / 256 * 256;
};
size_t gdn_mfma_record_bytes(int C, int d);

// 16-byte alignment check of a device pointer (NULL passes; checked elsewhere).
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_bytes(int32_t dt) { return dt == HLTA_BF16 ? 2 : 4; }

}  // namespace hlta
