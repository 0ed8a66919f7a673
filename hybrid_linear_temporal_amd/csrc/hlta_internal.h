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
  int gdn_G = 1;            // MFMA memory: segments per (batch row, head) run side by side
  int gdn_seg_chunks = 0;   //   and chunks per segment (the last may have fewer)
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
// aligned: per-row softmax statistics of both branches (two arrays); five
// d x d matrices per chunk of C = gdn_chunk tokens (transition, own state,
// own adjoint, start state, adjoint at the end); one
// slot per chunk for the memory's per-chunk kernels (the chunk's 64-row
// matrices, bwd_slot_floats(d) floats: those of the chunk's forward are formed
// once, by the first kernel, and read again by the last); partial sums of the
// mix-weight gradient.
constexpr int kBwdWorkgroups = 512;   // persistent grid of the memory's per-chunk kernels
// sixteen 64 x d and eight 64 x 64 fp32 matrices
constexpr size_t bwd_slot_floats(int d) { return 16 * size_t(64) * size_t(d) + 8 * size_t(64) * 64; }
constexpr int kDwSlices = 128;
struct BwdPlan {
  size_t stats_bytes = 0;   // each of the two: [2, B*L*H]
  size_t mat_off = 0, mat_bytes = 0;   // each of the five: [B*H*n_chunks, d, d]
  size_t slot_off = 0;
  int n_slots = 0;
  size_t slot_floats = 0;   // floats of one slot (one chunk's matrices in the memory's backward)
  size_t part_off = 0;
  size_t total = 0;
};
hlta_status make_bwd_plan(const hlta_config* cfg, BwdPlan* plan);

// Is there an MFMA kernel for this shape?
bool mfma_attn_supported(const hlta_config* cfg);
bool mfma_gdn_supported(const hlta_config* cfg);

// Per-chunk record sizes of the GDN scratch (in bytes).
size_t gdn_generic_record_bytes(int C, int d);

// Scratch of the MFMA memory kernels: one 13,056-byte record per chunk (the
// chunk's T'' = T diag(b) and T' = T diag(b gamma / ||k||) in bf16 operand
// order, then its gate prefix sums, b and inverse key norms), then, when G > 1,
// the segment maps:
// 2G - 1 d x d fp32 matrices per (batch row, head) (per segment but the last
// its N and M, and a copy of the start state).
size_t gdn_seg_record_bytes(int B, int H, long long n_chunks);
size_t gdn_seg_map_bytes(int B, int H, int G, int d);


// 16-byte alignment check of a device pointer (NULL passes; checked elsewhere).
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t dtype_bytes(int32_t dt) { return dt == HLTA_BF16 ? 2 : 4; }

}  // namespace hlta
