// HIP-free host layer of the HLTA library: status strings, the thread-local
// error message, config validation, kernel selection and workspace sizing.
// Built into libhlta.so and, with g++, into a CPU test binary.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <initializer_list>
#include <limits>
#include <string>

#include "hlta_internal.h"

namespace hlta {

static thread_local std::string g_last_error;

hlta_status fail(hlta_status s, const std::string& msg) {
  g_last_error = std::string(hlta_status_string(s)) + ": " + msg;
  return s;
}

void clear_error() { g_last_error.clear(); }

static bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *out = a * b;
  return true;
}

// product of non-negative factors, false if it leaves int64
static bool prod_ok(std::initializer_list<int64_t> f, int64_t* out) {
  int64_t x = 1;
  for (int64_t v : f)
    if (!mul_ok(x, v, &x)) return false;
  *out = x;
  return true;
}

static bool add_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0 || a > std::numeric_limits<int64_t>::max() - b) return false;
  *out = a + b;
  return true;
}

// x rounded up to a multiple of 256, false if it leaves int64
static bool align256_ok(int64_t x, int64_t* out) {
  if (x < 0 || x > std::numeric_limits<int64_t>::max() - 255) return false;
  *out = (x + 255) / 256 * 256;
  return true;
}

hlta_status check_config(const hlta_config* cfg) {
  if (!cfg) return fail(HLTA_E_NULL, "config is NULL");
  if (cfg->B < 1) return fail(HLTA_E_SHAPE, "B must be >= 1");
  if (cfg->H < 1) return fail(HLTA_E_SHAPE, "H must be >= 1");
  if (cfg->T < 0) return fail(HLTA_E_SHAPE, "T must be >= 0");
  if (cfg->P < 1) return fail(HLTA_E_SHAPE, "P must be >= 1");
  if (cfg->d != 32 && cfg->d != 64 && cfg->d != 128)
    return fail(HLTA_E_UNSUPPORTED, "d must be 32, 64 or 128 (got " + std::to_string(cfg->d) + ")");
  if (cfg->swa_frames < 0) return fail(HLTA_E_SHAPE, "swa_frames must be >= 0");
  if (cfg->dswa_dilation < 1) return fail(HLTA_E_SHAPE, "dswa_dilation must be >= 1");
  if (cfg->dswa_taps < 0) return fail(HLTA_E_SHAPE, "dswa_taps must be >= 0");
  if (cfg->gdn_chunk != 16 && cfg->gdn_chunk != 32 && cfg->gdn_chunk != 64)
    return fail(HLTA_E_UNSUPPORTED, "gdn_chunk must be 16, 32 or 64");
  if (!std::isfinite(cfg->softmax_scale)) return fail(HLTA_E_SHAPE, "softmax_scale is not finite");
  if (cfg->gdn_l2norm_qk != 0 && cfg->gdn_l2norm_qk != 1)
    return fail(HLTA_E_SHAPE, "gdn_l2norm_qk must be 0 or 1");
  const bool in_ok = cfg->in_dtype == HLTA_F32 || cfg->in_dtype == HLTA_BF16;
  const bool out_ok = cfg->out_dtype == HLTA_F32 || cfg->out_dtype == HLTA_BF16;
  if (!in_ok || !out_ok) return fail(HLTA_E_DTYPE, "dtype must be HLTA_F32 or HLTA_BF16");
  if (cfg->in_dtype == HLTA_F32 && cfg->out_dtype != HLTA_F32)
    return fail(HLTA_E_DTYPE, "float32 inputs need float32 outputs");
  if (cfg->impl != HLTA_IMPL_AUTO && cfg->impl != HLTA_IMPL_GENERIC && cfg->impl != HLTA_IMPL_MFMA)
    return fail(HLTA_E_SHAPE, "impl must be HLTA_IMPL_AUTO, _GENERIC or _MFMA");
  if (cfg->gate_logits != 0 && cfg->gate_logits != 1) return fail(HLTA_E_SHAPE, "gate_logits must be 0 or 1");
  if (!std::isfinite(cfg->rope_theta) || cfg->rope_theta < 0.f)
    return fail(HLTA_E_SHAPE, "rope_theta must be finite and >= 0");
  if (cfg->rope_theta > 0.f &&
      (cfg->rope_grid_h < 1 || cfg->rope_grid_w < 1 || int64_t(cfg->rope_grid_h) * cfg->rope_grid_w != cfg->P))
    return fail(HLTA_E_SHAPE, "rope_grid_h * rope_grid_w must equal P (" + std::to_string(cfg->rope_grid_h) +
                                  " x " + std::to_string(cfg->rope_grid_w) + " vs " + std::to_string(cfg->P) + ")");
  // every element offset must fit in int64, and token counts in int32 grids
  int64_t L, n;
  if (!mul_ok(cfg->T, cfg->P, &L) || !mul_ok(L, cfg->B, &n) || !mul_ok(n, cfg->H, &n) ||
      !mul_ok(n, cfg->d, &n))
    return fail(HLTA_E_SHAPE, "B*T*P*H*d overflows int64");
  if (L > (int64_t(1) << 31) - 1) return fail(HLTA_E_SHAPE, "T*P must be < 2^31");
  return HLTA_OK;
}

// the MFMA attention kernel addresses a 64-key tile from at most two frames
bool mfma_attn_supported(const hlta_config* cfg) {
  return cfg->in_dtype == HLTA_BF16 && cfg->d == 128 && cfg->P >= 64;
}

bool mfma_gdn_supported(const hlta_config* cfg) {
  return cfg->in_dtype == HLTA_BF16 && cfg->d == 128 && cfg->gdn_chunk == 64;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// generic record: W, U', Q*gamma, K*gamma_C/gamma [C x d] + Aqk [C x C] + gamma_C, fp32
size_t gdn_generic_record_bytes(int C, int d) {
  return align_up(sizeof(float) * (4 * size_t(C) * d + size_t(C) * C + 1), 256);
}

// one record per chunk: T'' and T' as six 1 KB operand tiles each, then 3 x 64 fp32 per-token values
size_t gdn_seg_record_bytes(int B, int H, long long n_chunks) { return size_t(B) * H * size_t(n_chunks) * 13056; }

size_t gdn_seg_map_bytes(int B, int H, int G, int d) {
  return G > 1 ? size_t(B) * H * (2 * size_t(G) - 1) * d * d * sizeof(float) : 0;
}

// Segments per (batch row, head) for the MFMA memory kernels: enough that the
// passes fill two workgroups on each of the 256 compute units, with at least
// four chunks per segment; one segment when the heads alone fill the chip.
static void gdn_segments(int64_t bh, int64_t n_chunks, int* G, int* seg_chunks) {
  int64_t g = 1;
  if (bh < 128) g = std::max<int64_t>(1, std::min<int64_t>(512 / bh, n_chunks / 4));
  const int64_t s = n_chunks > 0 ? (n_chunks + g - 1) / g : 1;
  *seg_chunks = int(s);
  *G = n_chunks > 0 ? int((n_chunks + s - 1) / s) : 1;
}

hlta_status make_plan(const hlta_config* cfg, int64_t L, Plan* plan) {
  hlta_status s = check_config(cfg);
  if (s != HLTA_OK) return s;
  Plan p;
  p.L = L;
  p.n_chunks = (L + cfg->gdn_chunk - 1) / cfg->gdn_chunk;
  p.scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / std::sqrt(float(cfg->d));
  const bool ma = mfma_attn_supported(cfg), mg = mfma_gdn_supported(cfg);
  switch (cfg->impl) {
    case HLTA_IMPL_GENERIC:
      p.attn = p.gdn = Impl::Generic;
      break;
    case HLTA_IMPL_MFMA:
      if (!ma || !mg)
        return fail(HLTA_E_UNSUPPORTED,
                    "MFMA kernels need bf16 inputs, d = 128, gdn_chunk = 64 and P >= 64");
      p.attn = p.gdn = Impl::Mfma;
      break;
    default:
      p.attn = ma ? Impl::Mfma : Impl::Generic;
      p.gdn = mg ? Impl::Mfma : Impl::Generic;
  }
  // the MFMA memory kernels address one batch row of q, k, v and the outputs
  // with 32-bit offsets
  if (p.gdn == Impl::Mfma && L * int64_t(cfg->H) * cfg->d * 4 > int64_t(0xFFFFFFFF)) {
    if (cfg->impl == HLTA_IMPL_MFMA)
      return fail(HLTA_E_UNSUPPORTED, "the MFMA memory kernels need L*H*d*4 < 2^32 bytes per batch row");
    p.gdn = Impl::Generic;
  }
  const int64_t bh = int64_t(cfg->B) * cfg->H;
  int64_t gdn = 0;
  if (p.gdn == Impl::Mfma) {
    gdn_segments(bh, p.n_chunks, &p.gdn_G, &p.gdn_seg_chunks);
    int64_t recs = 0, maps = 0;
    if (!prod_ok({bh, p.n_chunks, 13056}, &recs) ||
        !prod_ok({bh, p.gdn_G > 1 ? 2 * int64_t(p.gdn_G) - 1 : 0, int64_t(cfg->d) * cfg->d, 4}, &maps) ||
        !add_ok(recs, maps, &gdn))
      return fail(HLTA_E_SHAPE, "workspace size overflows int64");
    if (size_t(recs) != gdn_seg_record_bytes(cfg->B, cfg->H, p.n_chunks) ||
        size_t(maps) != gdn_seg_map_bytes(cfg->B, cfg->H, p.gdn_G, cfg->d))
      return fail(HLTA_E_SHAPE, "internal: memory workspace layout mismatch");
  } else {
    if (!prod_ok({bh, p.n_chunks, int64_t(gdn_generic_record_bytes(cfg->gdn_chunk, cfg->d))}, &gdn))
      return fail(HLTA_E_SHAPE, "workspace size overflows int64");
  }
  p.ws_gdn = size_t(gdn);
  p.ws_total = p.ws_gdn;
  if (cfg->rope_theta > 0.f) {
    // rotated q and k of the softmax branches, [B, L, H, d] in_dtype each
    int64_t n = 0, off = 0, total = 0;
    if (!prod_ok({bh, L, cfg->d, int64_t(dtype_bytes(cfg->in_dtype))}, &n) || !align256_ok(n, &n) ||
        !align256_ok(gdn, &off) || !add_ok(off, n, &total) || !add_ok(total, n, &total))
      return fail(HLTA_E_SHAPE, "workspace size overflows int64");
    p.ws_rope_bytes = size_t(n);
    p.ws_rope_off = size_t(off);
    p.ws_total = size_t(total);
  }
  *plan = p;
  return HLTA_OK;
}

hlta_status make_bwd_plan(const hlta_config* cfg, BwdPlan* plan) {
  hlta_status s = check_config(cfg);
  if (s != HLTA_OK) return s;
  const int64_t L = int64_t(cfg->T) * cfg->P, C = cfg->gdn_chunk, nch = (L + C - 1) / C;
  const int64_t dd = int64_t(cfg->d) * cfg->d, bh = int64_t(cfg->B) * cfg->H;
  BwdPlan p;
  if (bh * nch > std::numeric_limits<int>::max()) return fail(HLTA_E_SHAPE, "more than 2^31 - 1 chunks");
  p.n_slots = int(std::max<int64_t>(bh * nch, 1));
  int64_t stats = 0, mats = 0, mats5 = 0, slots = 0, part = 0, off = 0, total = 0;
  if (!prod_ok({bh, L, 2, 4}, &stats) || !align256_ok(stats, &stats) ||
      !prod_ok({bh, nch, dd, 4}, &mats) || !align256_ok(mats, &mats) || !mul_ok(mats, 5, &mats5) ||
      !prod_ok({p.n_slots, int64_t(bwd_slot_floats(cfg->d)), 4}, &slots) || !align256_ok(slots, &slots) ||
      !prod_ok({cfg->H, kDwSlices, 3, 4}, &part) || !align256_ok(part, &part) ||
      !add_ok(stats, stats, &off) || !add_ok(off, mats5, &off) || !add_ok(off, slots, &total) || !add_ok(total, part, &total))
    return fail(HLTA_E_SHAPE, "workspace size overflows int64");
  p.stats_bytes = size_t(stats);
  p.mat_off = 2 * p.stats_bytes;
  p.mat_bytes = size_t(mats);
  p.slot_off = p.mat_off + 5 * p.mat_bytes;
  p.slot_floats = bwd_slot_floats(cfg->d);
  p.part_off = p.slot_off + size_t(slots);
  p.total = size_t(total);
  *plan = p;
  return HLTA_OK;
}

}  // namespace hlta

using namespace hlta;

extern "C" {

int32_t hlta_abi_version(void) { return HLTA_ABI_VERSION; }

const char* hlta_status_string(int32_t s) {
  switch (s) {
    case HLTA_OK: return "HLTA_OK";
    case HLTA_E_NULL: return "HLTA_E_NULL";
    case HLTA_E_SHAPE: return "HLTA_E_SHAPE";
    case HLTA_E_DTYPE: return "HLTA_E_DTYPE";
    case HLTA_E_UNSUPPORTED: return "HLTA_E_UNSUPPORTED";
    case HLTA_E_WORKSPACE: return "HLTA_E_WORKSPACE";
    case HLTA_E_ALIGN: return "HLTA_E_ALIGN";
    case HLTA_E_STATE: return "HLTA_E_STATE";
    case HLTA_E_HIP: return "HLTA_E_HIP";
    default: return "HLTA_E_UNKNOWN";
  }
}

const char* hlta_last_error(void) { return g_last_error.c_str(); }

hlta_status hlta_validate_config(const hlta_config* cfg) {
  clear_error();
  return check_config(cfg);
}

size_t hlta_fwd_workspace_bytes(const hlta_config* cfg) {
  clear_error();
  Plan p;
  if (!cfg || make_plan(cfg, int64_t(cfg->T) * cfg->P, &p) != HLTA_OK) return 0;
  return p.ws_total;
}

size_t hlta_step_workspace_bytes(const hlta_config* cfg) {
  clear_error();
  Plan p;
  if (!cfg || make_plan(cfg, cfg->P, &p) != HLTA_OK) return 0;
  return p.ws_total;
}

size_t hlta_bwd_workspace_bytes(const hlta_config* cfg) {
  clear_error();
  BwdPlan p;
  if (!cfg || make_bwd_plan(cfg, &p) != HLTA_OK) return 0;
  return p.total;
}

size_t hlta_stream_ring_bytes(const hlta_config* cfg, int32_t ring_frames) {
  clear_error();
  if (check_config(cfg) != HLTA_OK) return 0;
  if (ring_frames < 1) {
    fail(HLTA_E_SHAPE, "ring_frames must be >= 1");
    return 0;
  }
  int64_t n = 0;
  if (!prod_ok({cfg->B, ring_frames, cfg->P, cfg->H, cfg->d, int64_t(dtype_bytes(cfg->in_dtype))}, &n)) {
    fail(HLTA_E_SHAPE, "ring size overflows int64");
    return 0;
  }
  return size_t(n);
}

}  // extern "C"
