// Host-side checks of the HLTA library's validation and planning layer
// (hlta_host.cpp), built with g++ together with that file under
// AddressSanitizer and UndefinedBehaviorSanitizer; no GPU and no HIP.
//
// 1. status strings and NULL handling;
// 2. the workloads the library is measured on: plans select the MFMA kernels,
//    segments cover the chunks, workspace sizes match the exported calls;
// 3. one invalid field at a time: the expected status and a message;
// 4. a seeded sweep over configs whose fields mix edge values (0, -1, the
//    int32 limits, sizes around the kernels' tile sizes, NaN and infinities):
//    every call returns, every accepted plan has a consistent layout, and a
//    refused one says why. The sanitizers turn any out-of-bounds access,
//    signed overflow or invalid conversion into a failure.
//
// Prints "host checks passed: <n> configs" and exits 0, or prints the first
// failure and exits 1.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>

#include "../../hybrid_linear_temporal_amd/csrc/hlta_internal.h"

using namespace hlta;

static int g_failures = 0;
static long g_accepted = 0, g_planned = 0;

#define CHECK(cond, ...)                                               \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                               \
      std::fprintf(stderr, "\n");                                      \
      ++g_failures;                                                    \
      return false;                                                    \
    }                                                                  \
  } while (0)

static hlta_config base_config() {
  hlta_config c;
  std::memset(&c, 0, sizeof(c));
  c.B = 1;
  c.H = 24;
  c.T = 31;
  c.P = 1560;
  c.d = 128;
  c.swa_frames = 3;
  c.dswa_dilation = 4;
  c.dswa_taps = 4;
  c.gdn_chunk = 64;
  c.softmax_scale = 0.f;
  c.gdn_l2norm_qk = 1;
  c.in_dtype = HLTA_BF16;
  c.out_dtype = HLTA_BF16;
  c.impl = HLTA_IMPL_AUTO;
  c.rope_theta = 0.f;
  c.gate_logits = 0;
  return c;
}

static std::string describe(const hlta_config& c) {
  char buf[512];
  std::snprintf(buf, sizeof(buf),
                "B=%d H=%d T=%d P=%d d=%d W=%d dil=%d taps=%d C=%d scale=%g l2=%d in=%d out=%d impl=%d "
                "rope=%g grid=%dx%d logits=%d",
                c.B, c.H, c.T, c.P, c.d, c.swa_frames, c.dswa_dilation, c.dswa_taps, c.gdn_chunk,
                double(c.softmax_scale), c.gdn_l2norm_qk, c.in_dtype, c.out_dtype, c.impl, double(c.rope_theta),
                c.rope_grid_h, c.rope_grid_w, c.gate_logits);
  return buf;
}

static bool message_names(hlta_status s) {
  const std::string msg = hlta_last_error();
  const std::string name = hlta_status_string(s);
  return msg.size() > name.size() + 2 && msg.compare(0, name.size(), name) == 0;
}

// Layout invariants of an accepted forward plan over L tokens per row.
static bool check_plan(const hlta_config& c, int64_t L, const Plan& p) {
  const std::string cs = describe(c);
  CHECK(p.L == L, "%s", cs.c_str());
  CHECK(p.n_chunks == (L + c.gdn_chunk - 1) / c.gdn_chunk, "%s", cs.c_str());
  CHECK(p.scale > 0.f && std::isfinite(p.scale), "%s", cs.c_str());
  if (c.softmax_scale > 0.f) CHECK(p.scale == c.softmax_scale, "%s", cs.c_str());
  CHECK(p.attn == Impl::Generic || p.attn == Impl::Mfma, "%s", cs.c_str());
  CHECK(p.gdn == Impl::Generic || p.gdn == Impl::Mfma, "%s", cs.c_str());
  if (p.attn == Impl::Mfma) CHECK(mfma_attn_supported(&c), "%s", cs.c_str());
  if (p.gdn == Impl::Mfma) {
    CHECK(mfma_gdn_supported(&c), "%s", cs.c_str());
    CHECK(p.gdn_G >= 1 && p.gdn_seg_chunks >= 1, "G=%d s=%d %s", p.gdn_G, p.gdn_seg_chunks, cs.c_str());
    if (p.n_chunks > 0) {
      // the segments cover the chunks, and none is empty
      CHECK(int64_t(p.gdn_G) * p.gdn_seg_chunks >= p.n_chunks, "G=%d s=%d %s", p.gdn_G, p.gdn_seg_chunks,
            cs.c_str());
      CHECK(int64_t(p.gdn_G - 1) * p.gdn_seg_chunks < p.n_chunks, "G=%d s=%d %s", p.gdn_G, p.gdn_seg_chunks,
            cs.c_str());
    }
    const size_t recs = gdn_seg_record_bytes(c.B, c.H, p.n_chunks);
    CHECK(p.ws_gdn == recs + gdn_seg_map_bytes(c.B, c.H, p.gdn_G, c.d), "%s", cs.c_str());
    CHECK(recs % 256 == 0, "%s", cs.c_str());
  } else {
    CHECK(p.ws_gdn == size_t(c.B) * size_t(c.H) * size_t(p.n_chunks) * gdn_generic_record_bytes(c.gdn_chunk, c.d),
          "%s", cs.c_str());
  }
  if (c.rope_theta > 0.f) {
    CHECK(p.ws_rope_off % 256 == 0 && p.ws_rope_off >= p.ws_gdn, "%s", cs.c_str());
    CHECK(p.ws_rope_bytes % 256 == 0, "%s", cs.c_str());
    CHECK(p.ws_rope_bytes >= size_t(c.B) * size_t(L) * size_t(c.H) * size_t(c.d) * dtype_bytes(c.in_dtype), "%s",
          cs.c_str());
    CHECK(p.ws_total == p.ws_rope_off + 2 * p.ws_rope_bytes, "%s", cs.c_str());
  } else {
    CHECK(p.ws_total == p.ws_gdn, "%s", cs.c_str());
  }
  return true;
}

static bool check_bwd_plan(const hlta_config& c, const BwdPlan& p) {
  const std::string cs = describe(c);
  const int64_t L = int64_t(c.T) * c.P, nch = (L + c.gdn_chunk - 1) / c.gdn_chunk;
  CHECK(p.n_slots == std::max<int64_t>(int64_t(c.B) * c.H * nch, 1), "%s", cs.c_str());
  CHECK(p.stats_bytes % 256 == 0 && p.mat_bytes % 256 == 0, "%s", cs.c_str());
  CHECK(p.stats_bytes >= size_t(c.B) * c.H * size_t(L) * 8, "%s", cs.c_str());
  CHECK(p.mat_bytes >= size_t(c.B) * c.H * size_t(nch) * c.d * c.d * 4, "%s", cs.c_str());
  CHECK(p.mat_off == 2 * p.stats_bytes, "%s", cs.c_str());
  CHECK(p.slot_off == p.mat_off + 5 * p.mat_bytes, "%s", cs.c_str());
  CHECK(p.slot_floats >= 16 * size_t(64) * c.d + 7 * size_t(64) * 64, "%s", cs.c_str());
  CHECK(p.part_off >= p.slot_off + size_t(p.n_slots) * p.slot_floats * 4, "%s", cs.c_str());
  CHECK(p.total >= p.part_off + size_t(c.H) * kDwSlices * 3 * 4 && p.total % 256 == 0, "%s", cs.c_str());
  return true;
}

// Every exported sizing call and the internal planners on one config.
static bool check_config_all(const hlta_config& c) {
  const std::string cs = describe(c);
  const hlta_status v = hlta_validate_config(&c);
  if (v != HLTA_OK) {
    CHECK(message_names(v), "status %d message '%s' for %s", int(v), hlta_last_error(), cs.c_str());
    CHECK(hlta_fwd_workspace_bytes(&c) == 0, "%s", cs.c_str());
    CHECK(hlta_step_workspace_bytes(&c) == 0, "%s", cs.c_str());
    CHECK(hlta_bwd_workspace_bytes(&c) == 0, "%s", cs.c_str());
    CHECK(hlta_stream_ring_bytes(&c, 4) == 0, "%s", cs.c_str());
    return true;
  }
  CHECK(std::strlen(hlta_last_error()) == 0, "%s", cs.c_str());
  ++g_accepted;
  for (int step = 0; step < 2; ++step) {
    const int64_t L = step ? int64_t(c.P) : int64_t(c.T) * c.P;
    Plan p;
    const hlta_status s = make_plan(&c, L, &p);
    const size_t exported = step ? hlta_step_workspace_bytes(&c) : hlta_fwd_workspace_bytes(&c);
    if (s == HLTA_OK) {
      ++g_planned;
      if (!check_plan(c, L, p)) return false;
      CHECK(exported == p.ws_total, "%zu vs %zu %s", exported, p.ws_total, cs.c_str());
    } else {
      CHECK(s == HLTA_E_SHAPE || s == HLTA_E_UNSUPPORTED, "status %d %s", int(s), cs.c_str());
      CHECK(message_names(s), "'%s' %s", hlta_last_error(), cs.c_str());
      CHECK(exported == 0, "%s", cs.c_str());
    }
  }
  BwdPlan bp;
  const hlta_status sb = make_bwd_plan(&c, &bp);
  if (sb == HLTA_OK) {
    if (!check_bwd_plan(c, bp)) return false;
    CHECK(hlta_bwd_workspace_bytes(&c) == bp.total, "%s", cs.c_str());
  } else {
    CHECK(sb == HLTA_E_SHAPE && message_names(sb), "'%s' %s", hlta_last_error(), cs.c_str());
  }
  for (int32_t r : {-1, 0, 1, 17, std::numeric_limits<int32_t>::max()}) {
    const size_t n = hlta_stream_ring_bytes(&c, r);
    if (r < 1) {
      CHECK(n == 0 && message_names(HLTA_E_SHAPE), "ring %d %s", r, cs.c_str());
    } else {
      // the exact size in 128 bits: refused exactly when it leaves int64
      const unsigned __int128 want = (unsigned __int128)c.B * unsigned(r) * unsigned(c.P) * unsigned(c.H) *
                                     unsigned(c.d) * dtype_bytes(c.in_dtype);
      if (want > (unsigned __int128)std::numeric_limits<int64_t>::max())
        CHECK(n == 0 && message_names(HLTA_E_SHAPE), "ring %d '%s' %s", r, hlta_last_error(), cs.c_str());
      else
        CHECK(n == size_t(want), "ring %d %s", r, cs.c_str());
    }
  }
  return true;
}

static bool status_strings() {
  const char* names[] = {"HLTA_OK",    "HLTA_E_NULL",  "HLTA_E_SHAPE", "HLTA_E_DTYPE", "HLTA_E_UNSUPPORTED",
                         "HLTA_E_WORKSPACE", "HLTA_E_ALIGN", "HLTA_E_STATE", "HLTA_E_HIP"};
  for (int s = 0; s <= 8; ++s) CHECK(std::strcmp(hlta_status_string(s), names[s]) == 0, "status %d", s);
  for (int s : {-1, 9, 1000, std::numeric_limits<int32_t>::min()})
    CHECK(std::strcmp(hlta_status_string(s), "HLTA_E_UNKNOWN") == 0, "status %d", s);
  CHECK(hlta_abi_version() == HLTA_ABI_VERSION, "abi");
  CHECK(hlta_validate_config(nullptr) == HLTA_E_NULL && message_names(HLTA_E_NULL), "NULL config");
  CHECK(hlta_fwd_workspace_bytes(nullptr) == 0 && hlta_step_workspace_bytes(nullptr) == 0, "NULL sizing");
  CHECK(hlta_bwd_workspace_bytes(nullptr) == 0 && hlta_stream_ring_bytes(nullptr, 4) == 0, "NULL sizing");
  return true;
}

static bool workloads() {
  struct W { int B, T, P; };
  // 480P and 720P clips, the 8-rollout stream, a ragged small case
  const W ws[] = {{1, 31, 1560}, {1, 61, 1560}, {1, 61, 3600}, {8, 16, 1560}, {2, 3, 100}};
  for (const W& w : ws) {
    hlta_config c = base_config();
    c.B = w.B;
    c.T = w.T;
    c.P = w.P;
    if (!check_config_all(c)) return false;
    Plan p;
    CHECK(make_plan(&c, int64_t(c.T) * c.P, &p) == HLTA_OK, "%s", describe(c).c_str());
    CHECK(p.attn == Impl::Mfma && p.gdn == Impl::Mfma, "%s", describe(c).c_str());
    // rotary embedding on, over the frame's token grid
    for (int gh = 1; gh <= c.P; ++gh)
      if (c.P % gh == 0 && gh * gh >= c.P) {
        c.rope_theta = 10000.f;
        c.rope_grid_h = gh;
        c.rope_grid_w = c.P / gh;
        break;
      }
    if (!check_config_all(c)) return false;
  }
  // 480P / 31 frames: 756 chunks per head in 21 segments of 36
  hlta_config c = base_config();
  Plan p;
  CHECK(make_plan(&c, int64_t(c.T) * c.P, &p) == HLTA_OK, "480P");
  CHECK(p.n_chunks == 756 && p.gdn_G == 21 && p.gdn_seg_chunks == 36, "n=%lld G=%d s=%d",
        (long long)p.n_chunks, p.gdn_G, p.gdn_seg_chunks);
  CHECK(p.ws_total == size_t(24) * 756 * 13056 + size_t(24) * 41 * 128 * 128 * 4, "ws %zu", p.ws_total);
  return true;
}

static bool one_field_invalid() {
  struct Case {
    const char* what;
    void (*set)(hlta_config&);
    hlta_status want;
  };
  const Case cases[] = {
      {"B = 0", [](hlta_config& c) { c.B = 0; }, HLTA_E_SHAPE},
      {"H = -1", [](hlta_config& c) { c.H = -1; }, HLTA_E_SHAPE},
      {"T = -1", [](hlta_config& c) { c.T = -1; }, HLTA_E_SHAPE},
      {"P = 0", [](hlta_config& c) { c.P = 0; }, HLTA_E_SHAPE},
      {"d = 96", [](hlta_config& c) { c.d = 96; }, HLTA_E_UNSUPPORTED},
      {"W = -1", [](hlta_config& c) { c.swa_frames = -1; }, HLTA_E_SHAPE},
      {"dil = 0", [](hlta_config& c) { c.dswa_dilation = 0; }, HLTA_E_SHAPE},
      {"taps = -2", [](hlta_config& c) { c.dswa_taps = -2; }, HLTA_E_SHAPE},
      {"C = 48", [](hlta_config& c) { c.gdn_chunk = 48; }, HLTA_E_UNSUPPORTED},
      {"scale NaN", [](hlta_config& c) { c.softmax_scale = std::nanf(""); }, HLTA_E_SHAPE},
      {"scale inf", [](hlta_config& c) { c.softmax_scale = INFINITY; }, HLTA_E_SHAPE},
      {"l2norm 2", [](hlta_config& c) { c.gdn_l2norm_qk = 2; }, HLTA_E_SHAPE},
      {"in dtype 5", [](hlta_config& c) { c.in_dtype = 5; }, HLTA_E_DTYPE},
      {"f32 in, bf16 out", [](hlta_config& c) { c.in_dtype = HLTA_F32; }, HLTA_E_DTYPE},
      {"impl 3", [](hlta_config& c) { c.impl = 3; }, HLTA_E_SHAPE},
      {"gate_logits -1", [](hlta_config& c) { c.gate_logits = -1; }, HLTA_E_SHAPE},
      {"rope theta -1", [](hlta_config& c) { c.rope_theta = -1.f; }, HLTA_E_SHAPE},
      {"rope grid mismatch", [](hlta_config& c) { c.rope_theta = 1e4f; c.rope_grid_h = 30; c.rope_grid_w = 51; },
       HLTA_E_SHAPE},
      {"rope grid overflow",
       [](hlta_config& c) { c.rope_theta = 1e4f; c.rope_grid_h = 65536; c.rope_grid_w = 65536 + 1560; },
       HLTA_E_SHAPE},
      {"T*P >= 2^31", [](hlta_config& c) { c.H = 1; c.d = 32; c.T = 1 << 20; c.P = 1 << 12; }, HLTA_E_SHAPE},
      {"elements overflow int64",
       [](hlta_config& c) { c.B = std::numeric_limits<int32_t>::max(); c.H = c.B; c.T = c.B; c.P = c.B; },
       HLTA_E_SHAPE},
  };
  for (const Case& k : cases) {
    hlta_config c = base_config();
    k.set(c);
    const hlta_status s = hlta_validate_config(&c);
    CHECK(s == k.want, "%s: got %d want %d ('%s')", k.what, int(s), int(k.want), hlta_last_error());
    CHECK(message_names(s), "%s: message '%s'", k.what, hlta_last_error());
    if (!check_config_all(c)) return false;
  }
  // forcing the MFMA family where it has no kernel is refused, not downgraded
  hlta_config c = base_config();
  c.impl = HLTA_IMPL_MFMA;
  c.d = 64;
  Plan p;
  CHECK(make_plan(&c, 100, &p) == HLTA_E_UNSUPPORTED && message_names(HLTA_E_UNSUPPORTED), "MFMA forced, d = 64");
  return true;
}

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014)
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
  uint64_t z = (g_rng += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static int32_t draw_int(int32_t typical_lo, int32_t typical_hi) {
  static const int32_t edges[] = {std::numeric_limits<int32_t>::min(), -65, -1, 0, 1, 2, 3, 4, 15, 16, 17,
                                  31, 32, 33, 63, 64, 65, 96, 127, 128, 129, 1560, 3600, 65535, 1 << 20,
                                  1 << 30, std::numeric_limits<int32_t>::max()};
  const uint64_t r = next_u64();
  if (r % 12 == 0) return edges[(r >> 8) % (sizeof(edges) / sizeof(edges[0]))];
  return typical_lo + int32_t((r >> 8) % uint64_t(int64_t(typical_hi) - typical_lo + 1));
}

static float draw_float() {
  static const float vals[] = {std::nanf(""), INFINITY, -INFINITY, -1.f, 0.f, 1e-3f, 0.0883883f, 1.f, 1e4f, 3e38f};
  return vals[next_u64() % (sizeof(vals) / sizeof(vals[0]))];
}

static bool sweep(int n) {
  for (int i = 0; i < n; ++i) {
    hlta_config c;
    c.B = draw_int(1, 8);
    c.H = draw_int(1, 32);
    c.T = draw_int(0, 64);
    c.P = draw_int(1, 4000);
    const int32_t ds[] = {32, 64, 128};
    c.d = (next_u64() % 8) ? ds[next_u64() % 3] : draw_int(0, 256);
    c.swa_frames = draw_int(0, 8);
    c.dswa_dilation = draw_int(1, 8);
    c.dswa_taps = draw_int(0, 8);
    const int32_t cs[] = {16, 32, 64};
    c.gdn_chunk = (next_u64() % 8) ? cs[next_u64() % 3] : draw_int(0, 128);
    c.softmax_scale = draw_float();
    c.gdn_l2norm_qk = draw_int(0, 1);
    c.in_dtype = draw_int(0, 1);
    c.out_dtype = draw_int(0, 1);
    c.impl = draw_int(0, 2);
    c.rope_theta = (next_u64() % 2) ? 0.f : draw_float();
    c.rope_grid_h = draw_int(1, 64);
    c.rope_grid_w = (next_u64() % 2 && c.rope_grid_h > 0 && c.P % c.rope_grid_h == 0) ? c.P / c.rope_grid_h
                                                                                         : draw_int(1, 64);
    c.gate_logits = draw_int(0, 1);
    if (!check_config_all(c)) return false;
  }
  return true;
}

int main() {
  const int n_sweep = 200000;
  if (!status_strings() || !workloads() || !one_field_invalid() || !sweep(n_sweep)) {
    std::fprintf(stderr, "host checks FAILED (%d)\n", g_failures);
    return 1;
  }
  std::printf("host checks passed: %d configs (%ld accepted, %ld forward plans)\n", n_sweep, g_accepted,
              g_planned);
  return 0;
}
