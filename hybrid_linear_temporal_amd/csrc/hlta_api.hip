// C-ABI entry points that launch work: hlta_fwd (and its allocation-free
// variant hlta_fwd_noalloc), hlta_gdn_fwd, hlta_attn_fwd, the FP8 pair,
// hlta_bwd, hlta_stream_load_prefix, hlta_step_frame(_rollouts). Validation
// happens on the host before any launch; the library allocates no device
// memory (scratch is the caller's workspace, or for hlta_fwd_noalloc a fixed
// device array).
#include <mutex>
#include <string>

#include "hlta_device.h"
#include "hlta_internal.h"
#include "hlta_launch.h"

using namespace hlta;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

hlta_status hip_fail(hipError_t e, const char* what) {
  return fail(HLTA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

hlta_status need(const void* p, const char* name) {
  if (!p) return fail(HLTA_E_NULL, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(HLTA_E_ALIGN, std::string(name) + " is not 16-byte aligned");
  return HLTA_OK;
}

hlta_status maybe(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(HLTA_E_ALIGN, std::string(name) + " is not 16-byte aligned");
  return HLTA_OK;
}

#define HLTA_TRY(x)                  \
  do {                               \
    hlta_status s_ = (x);            \
    if (s_ != HLTA_OK) return s_;    \
  } while (0)

hlta_status check_outputs(const float* a, const float* b, const float* mix_w, void* o_swa, void* o_dswa,
                          void* o_gdn, void* o_mix) {
  HLTA_TRY(need(a, "a"));
  HLTA_TRY(need(b, "b"));
  HLTA_TRY(need(mix_w, "mix_w"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(need(o_mix, "o_mix"));
  return HLTA_OK;
}

// The mix's operands when it follows the memory branch (o_swa, o_dswa as
// already stored by the softmax branches).
struct MixOut {
  const void* swa;
  const void* dswa;
  void* out;
  const float* w;
};

// The memory branch; with mix set, the mix kernel after it. (Forming the mix
// in the memory's output pass instead was slower: its scattered 8-byte loads
// and stores of the branch outputs cost that pass more than the mix kernel's
// 16-byte streams take.)
hlta_status run_gdn(const hlta_config* cfg, const Plan& plan, const void* q, const void* k, const void* v,
                    const float* a, const float* b, const float* S0, float* S_out, void* o_gdn, void* workspace,
                    hipStream_t st, unsigned long long skip = 0, const MixOut* mix = nullptr) {
  GdnParams g{};
  g.skip = skip;
  g.q = q;
  g.k = k;
  g.v = v;
  g.a = a;
  g.b = b;
  g.S0 = S0;
  g.S_out = S_out;
  g.o = o_gdn;
  g.ws = static_cast<unsigned char*>(workspace);
  g.rec_bytes = plan.gdn == Impl::Mfma ? 0 : gdn_generic_record_bytes(cfg->gdn_chunk, cfg->d);
  g.B = cfg->B;
  g.H = cfg->H;
  g.L = plan.L;
  g.n_chunks = int(plan.n_chunks);
  g.l2norm = cfg->gdn_l2norm_qk;
  g.gate_logits = cfg->gate_logits;
  hipError_t e = plan.gdn == Impl::Mfma
                     ? launch_gdn_seg(g, plan.gdn_G, plan.gdn_seg_chunks, workspace, cfg->out_dtype, st)
                     : launch_gdn_generic(g, cfg->d, cfg->gdn_chunk, cfg->in_dtype, cfg->out_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "gated delta rule launch");
  if (mix) {
    e = launch_mix(mix->swa, mix->dswa, o_gdn, mix->out, mix->w, (long long)cfg->B * plan.L, cfg->H, cfg->d,
                   cfg->out_dtype, st, skip, plan.L);
    if (e != hipSuccess) return hip_fail(e, "mix launch");
  }
  return HLTA_OK;
}

hlta_status run_attn(const hlta_config* cfg, const Plan& plan, AttnParams attn, hipStream_t st) {
  attn.scale_log2 = plan.scale * kLog2e;
  hipError_t e = plan.attn == Impl::Mfma
                     ? launch_attn_mfma(attn, cfg->out_dtype, st)
                     : launch_attn_generic(attn, cfg->d, cfg->in_dtype, cfg->out_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return HLTA_OK;
}

hlta_status run_mix(const hlta_config* cfg, const Plan& plan, const void* o_swa, const void* o_dswa,
                    const void* o_gdn, void* o_mix, const float* mix_w, hipStream_t st, unsigned long long skip = 0) {
  hipError_t e = launch_mix(o_swa, o_dswa, o_gdn, o_mix, mix_w, (long long)cfg->B * plan.L, cfg->H, cfg->d,
                            cfg->out_dtype, st, skip, plan.L);
  if (e != hipSuccess) return hip_fail(e, "mix launch");
  return HLTA_OK;
}

// Rotary embedding on: rotate q and k of the softmax branches into the
// workspace (positions from attn.f0 or attn.ro) and point attn at the copies.
hlta_status run_rope(const hlta_config* cfg, const Plan& plan, AttnParams& attn, void* workspace, hipStream_t st) {
  if (cfg->rope_theta <= 0.f) return HLTA_OK;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  void* qr = ws + plan.ws_rope_off;
  void* kr = ws + plan.ws_rope_off + plan.ws_rope_bytes;
  hipError_t e = launch_rope_qk(attn.q, attn.k, qr, kr, cfg->B, plan.L, cfg->H, cfg->d, cfg->P, cfg->rope_grid_w,
                                cfg->rope_theta, cfg->in_dtype, attn.f0, attn.per_rollout, attn.ro, st);
  if (e != hipSuccess) return hip_fail(e, "rotary embedding launch");
  attn.q = qr;
  attn.k = kr;
  return HLTA_OK;
}

// One layer: the softmax branches, then the memory branch (GDN over L tokens
// per row) and the per-head mix of the three outputs, in order on st.
// Rollouts in attn.ro.skip are left out of all of it.
// (Running the two halves on two streams gains nothing here: the memory's
// passes need most of a compute unit's LDS per workgroup, so they cannot
// share the chip with the attention branches.) attn.* query fields set by caller.
hlta_status run_layer(const hlta_config* cfg, const Plan& plan, const void* q, const void* k, const void* v,
                      const float* a, const float* b, const float* S0, float* S_out, void* o_gdn,
                      const float* mix_w, void* o_mix, void* workspace, AttnParams& attn, hipStream_t st) {
  HLTA_TRY(run_rope(cfg, plan, attn, workspace, st));
  HLTA_TRY(run_attn(cfg, plan, attn, st));
  const MixOut mix{attn.o_swa, attn.o_dswa, o_mix, mix_w};
  return run_gdn(cfg, plan, q, k, v, a, b, S0, S_out, o_gdn, workspace, st, attn.ro.skip, &mix);
}

AttnParams full_attn_params(const hlta_config* cfg, const void* q, const void* k, const void* v, void* o_swa,
                            void* o_dswa) {
  AttnParams at{};
  at.q = q;
  at.k = k;
  at.v = v;
  at.o_swa = o_swa;
  at.o_dswa = o_dswa;
  at.B = cfg->B;
  at.H = cfg->H;
  at.T = cfg->T;
  at.P = cfg->P;
  at.W = cfg->swa_frames;
  at.dil = cfg->dswa_dilation;
  at.taps = cfg->dswa_taps;
  at.R = 0;
  at.f0 = 0;
  return at;
}

hlta_status check_workspace(const Plan& plan, const void* workspace, size_t ws_bytes) {
  if (plan.ws_total > 0) {
    HLTA_TRY(need(workspace, "workspace"));
    if (ws_bytes < plan.ws_total)
      return fail(HLTA_E_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                        std::to_string(plan.ws_total));
  }
  return HLTA_OK;
}

size_t state_bytes(const hlta_config* cfg) { return size_t(cfg->B) * cfg->H * cfg->d * cfg->d * sizeof(float); }

hlta_status fwd_body(const hlta_config* cfg, const Plan& plan, const void* q, const void* k, const void* v,
                     const float* a, const float* b, const float* mix_w, const float* S0, void* o_swa,
                     void* o_dswa, void* o_gdn, void* o_mix, float* S_out, void* workspace, size_t ws_bytes,
                     hipStream_t st);

// Scratch of hlta_fwd_noalloc: a fixed device array, one copy per GPU, held
// until the process ends. Host code never passes the array's name to a kernel
// (on the host it is only a stand-in for the symbol): the device address of
// each GPU's copy is looked up once, with that device current, and kept.
constexpr size_t kScratchBytes = HLTA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
hlta_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HLTA_E_UNSUPPORTED, "device " + std::to_string(dev) + " is beyond the " +
                                        std::to_string(kMaxDevices) + " devices the scratch table holds");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "scratch address lookup");
    if (!ptr) return fail(HLTA_E_HIP, "scratch address lookup returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HLTA_OK;
}

}  // namespace

extern "C" {

hlta_status hlta_fwd(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                     const float* b, const float* mix_w, const float* S0, void* o_swa, void* o_dswa,
                     void* o_gdn, void* o_mix, float* S_out, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  return fwd_body(cfg, plan, q, k, v, a, b, mix_w, S0, o_swa, o_dswa, o_gdn, o_mix, S_out, workspace, ws_bytes,
                  static_cast<hipStream_t>(stream));
}

hlta_status hlta_fwd_noalloc(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* mix_w, const float* S0, void* o_swa, void* o_dswa,
                             void* o_gdn, void* o_mix, float* S_out, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  if (plan.ws_total > kScratchBytes)
    return fail(HLTA_E_WORKSPACE, "this call needs " + std::to_string(plan.ws_total) +
                                      " bytes of scratch; the allocation-free entry point holds at most " +
                                      std::to_string(kScratchBytes) + " (use hlta_fwd with a workspace)");
  void* scratch_ptr = nullptr;
  if (plan.L > 0 && plan.ws_total > 0) HLTA_TRY(device_scratch(&scratch_ptr));
  return fwd_body(cfg, plan, q, k, v, a, b, mix_w, S0, o_swa, o_dswa, o_gdn, o_mix, S_out, scratch_ptr,
                  kScratchBytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// hlta_fwd after the config is checked and planned: argument checks, then the
// launches (shared by hlta_fwd and hlta_fwd_noalloc).
hlta_status fwd_body(const hlta_config* cfg, const Plan& plan, const void* q, const void* k, const void* v,
                     const float* a, const float* b, const float* mix_w, const float* S0, void* o_swa,
                     void* o_dswa, void* o_gdn, void* o_mix, float* S_out, void* workspace, size_t ws_bytes,
                     hipStream_t st) {
  HLTA_TRY(maybe(S0, "S0"));
  HLTA_TRY(maybe(S_out, "S_out"));
  if (plan.L == 0) {
    // empty clip: the state passes through unchanged
    if (S_out && S_out != S0) {
      hipError_t e = launch_copy_or_zero(S_out, S0, state_bytes(cfg), st);
      if (e != hipSuccess) return hip_fail(e, "state copy");
    }
    return HLTA_OK;
  }
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(check_outputs(a, b, mix_w, o_swa, o_dswa, o_gdn, o_mix));
  HLTA_TRY(check_workspace(plan, workspace, ws_bytes));
  AttnParams at = full_attn_params(cfg, q, k, v, o_swa, o_dswa);
  return run_layer(cfg, plan, q, k, v, a, b, S0, S_out, o_gdn, mix_w, o_mix, workspace, at, st);
}

}  // namespace

extern "C" {

hlta_status hlta_gdn_fwd(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* S0, void* o_gdn, float* S_out, void* workspace,
                         size_t ws_bytes, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  HLTA_TRY(maybe(S0, "S0"));
  HLTA_TRY(maybe(S_out, "S_out"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.L == 0) {
    if (S_out && S_out != S0) {
      hipError_t e = launch_copy_or_zero(S_out, S0, state_bytes(cfg), st);
      if (e != hipSuccess) return hip_fail(e, "state copy");
    }
    return HLTA_OK;
  }
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(a, "a"));
  HLTA_TRY(need(b, "b"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(check_workspace(plan, workspace, ws_bytes));
  return run_gdn(cfg, plan, q, k, v, a, b, S0, S_out, o_gdn, workspace, st);
}

hlta_status hlta_attn_fwd(const hlta_config* cfg, const void* q, const void* k, const void* v,
                          const float* mix_w, const void* o_gdn, void* o_swa, void* o_dswa, void* o_mix,
                          void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  if (plan.L == 0) return HLTA_OK;
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(mix_w, "mix_w"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  HLTA_TRY(need(o_mix, "o_mix"));
  if (cfg->rope_theta > 0.f)
    return fail(HLTA_E_UNSUPPORTED, "the rotary embedding needs a workspace: use hlta_fwd");
  AttnParams at = full_attn_params(cfg, q, k, v, o_swa, o_dswa);
  hipStream_t st = static_cast<hipStream_t>(stream);
  HLTA_TRY(run_attn(cfg, plan, at, st));
  return run_mix(cfg, plan, o_swa, o_dswa, o_gdn, o_mix, mix_w, st);
}

hlta_status hlta_attn_branches(const hlta_config* cfg, const void* q, const void* k, const void* v, void* o_swa,
                               void* o_dswa, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  if (plan.L == 0) return HLTA_OK;
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  if (cfg->rope_theta > 0.f)
    return fail(HLTA_E_UNSUPPORTED, "the rotary embedding needs a workspace: use hlta_fwd");
  AttnParams at = full_attn_params(cfg, q, k, v, o_swa, o_dswa);
  return run_attn(cfg, plan, at, static_cast<hipStream_t>(stream));
}

hlta_status hlta_gdn_mix_fwd(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                             const float* b, const float* mix_w, const float* S0, const void* o_swa,
                             const void* o_dswa, void* o_gdn, void* o_mix, float* S_out, void* workspace,
                             size_t ws_bytes, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  HLTA_TRY(maybe(S0, "S0"));
  HLTA_TRY(maybe(S_out, "S_out"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.L == 0) {
    if (S_out && S_out != S0) {
      hipError_t e = launch_copy_or_zero(S_out, S0, state_bytes(cfg), st);
      if (e != hipSuccess) return hip_fail(e, "state copy");
    }
    return HLTA_OK;
  }
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(a, "a"));
  HLTA_TRY(need(b, "b"));
  HLTA_TRY(need(mix_w, "mix_w"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(need(o_mix, "o_mix"));
  HLTA_TRY(check_workspace(plan, workspace, ws_bytes));
  const MixOut mix{o_swa, o_dswa, o_mix, mix_w};
  return run_gdn(cfg, plan, q, k, v, a, b, S0, S_out, o_gdn, workspace, st, 0, &mix);
}

hlta_status hlta_attn_fwd_lse(const hlta_config* cfg, const void* q, const void* k, const void* v,
                              const float* mix_w, const void* o_gdn, void* o_swa, void* o_dswa, void* o_mix,
                              float* lse, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  if (plan.L == 0) return HLTA_OK;
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(mix_w, "mix_w"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  HLTA_TRY(need(o_mix, "o_mix"));
  HLTA_TRY(need(lse, "lse"));
  if (cfg->rope_theta > 0.f)
    return fail(HLTA_E_UNSUPPORTED, "the rotary embedding needs a workspace: use hlta_fwd");
  AttnParams at = full_attn_params(cfg, q, k, v, o_swa, o_dswa);
  at.lse = lse;
  hipStream_t st = static_cast<hipStream_t>(stream);
  HLTA_TRY(run_attn(cfg, plan, at, st));
  return run_mix(cfg, plan, o_swa, o_dswa, o_gdn, o_mix, mix_w, st);
}

hlta_status hlta_quantize_fp8(const hlta_config* cfg, const void* q, const void* k, const void* v, void* q8,
                              void* k8, void* v8, float* scales, void* stream) {
  clear_error();
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(need(q, "q"));
  HLTA_TRY(need(k, "k"));
  HLTA_TRY(need(v, "v"));
  HLTA_TRY(need(q8, "q8"));
  HLTA_TRY(need(k8, "k8"));
  HLTA_TRY(need(v8, "v8"));
  HLTA_TRY(need(scales, "scales"));
  const long long L = (long long)cfg->T * cfg->P;
  hipError_t e = launch_quantize_e4m3(q, k, v, q8, k8, v8, scales, cfg->B, L, cfg->H, cfg->d, cfg->in_dtype,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quantisation launch");
  return HLTA_OK;
}

hlta_status hlta_attn_fwd_fp8(const hlta_config* cfg, const void* q8, const void* k8, const void* v8,
                              const float* scales, const float* mix_w, const void* o_gdn, void* o_swa,
                              void* o_dswa, void* o_mix, void* stream) {
  clear_error();
  Plan plan;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  if (cfg->d != 128 || cfg->P < 64)
    return fail(HLTA_E_UNSUPPORTED, "the FP8 softmax branches need d = 128 and P >= 64");
  if (cfg->rope_theta > 0.f)
    return fail(HLTA_E_UNSUPPORTED, "the FP8 softmax branches take codes of already rotated q and k");
  if (plan.L == 0) return HLTA_OK;
  HLTA_TRY(need(q8, "q8"));
  HLTA_TRY(need(k8, "k8"));
  HLTA_TRY(need(v8, "v8"));
  HLTA_TRY(need(scales, "scales"));
  HLTA_TRY(need(mix_w, "mix_w"));
  HLTA_TRY(need(o_gdn, "o_gdn"));
  HLTA_TRY(need(o_swa, "o_swa"));
  HLTA_TRY(need(o_dswa, "o_dswa"));
  HLTA_TRY(need(o_mix, "o_mix"));
  AttnParams at = full_attn_params(cfg, q8, k8, v8, o_swa, o_dswa);
  at.scale_log2 = plan.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_attn_fp8(at, scales, cfg->out_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "FP8 attention launch");
  return run_mix(cfg, plan, o_swa, o_dswa, o_gdn, o_mix, mix_w, st);
}

}  // extern "C"

// hlta_bwd, with the softmax row statistics given (lse, from
// hlta_attn_fwd_lse) or recomputed (lse NULL).
static hlta_status bwd_impl(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                            const float* b, const float* mix_w, const float* S0, const void* o_swa,
                            const void* o_dswa, const void* o_gdn, const void* d_mix, float* dq, float* dk,
                            float* dv, float* da, float* db, float* dmix_w, float* dS0, const float* lse,
                            void* workspace, size_t ws_bytes, void* stream) {
  Plan plan;
  BwdPlan bp;
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(make_plan(cfg, int64_t(cfg->T) * cfg->P, &plan));
  HLTA_TRY(make_bwd_plan(cfg, &bp));
  if (cfg->rope_theta > 0.f) return fail(HLTA_E_UNSUPPORTED, "the backward takes no rotary embedding");
  if (cfg->gate_logits) return fail(HLTA_E_UNSUPPORTED, "the backward takes the gates themselves, not logits");
  HLTA_TRY(maybe(S0, "S0"));
  HLTA_TRY(maybe(dS0, "dS0"));
  HLTA_TRY(need(dmix_w, "dmix_w"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.L == 0) {
    // no tokens: every gradient that exists is zero
    hipError_t e = launch_copy_or_zero(dmix_w, nullptr, size_t(cfg->H) * 3 * sizeof(float), st);
    if (e == hipSuccess && dS0) e = launch_copy_or_zero(dS0, nullptr, state_bytes(cfg), st);
    if (e != hipSuccess) return hip_fail(e, "gradient clear");
    return HLTA_OK;
  }
  const void* ins[] = {q, k, v, a, b, mix_w, o_swa, o_dswa, o_gdn, d_mix, dq, dk, dv, da, db};
  const char* names[] = {"q", "k", "v", "a", "b", "mix_w", "o_swa", "o_dswa", "o_gdn", "d_mix",
                         "dq", "dk", "dv", "da", "db"};
  for (int i = 0; i < 15; ++i) HLTA_TRY(need(ins[i], names[i]));
  HLTA_TRY(need(workspace, "workspace"));
  if (ws_bytes < bp.total)
    return fail(HLTA_E_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                      std::to_string(bp.total));
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  BwdArgs x{};
  x.attn = full_attn_params(cfg, q, k, v, nullptr, nullptr);
  x.attn.scale_log2 = plan.scale * kLog2e;
  x.gdn.q = q;
  x.gdn.k = k;
  x.gdn.v = v;
  x.gdn.a = a;
  x.gdn.b = b;
  x.gdn.S0 = S0;
  x.gdn.B = cfg->B;
  x.gdn.H = cfg->H;
  x.gdn.L = plan.L;
  x.gdn.n_chunks = int(plan.n_chunks);
  x.gdn.l2norm = cfg->gdn_l2norm_qk;
  x.d_mix = d_mix;
  x.mix_w = mix_w;
  x.o_swa = o_swa;
  x.o_dswa = o_dswa;
  x.o_gdn = o_gdn;
  x.dq = dq;
  x.dk = dk;
  x.dv = dv;
  x.da = da;
  x.db = db;
  x.dmix_w = dmix_w;
  x.dS0 = dS0;
  x.lse2 = reinterpret_cast<float*>(ws);
  x.dsum = reinterpret_cast<float*>(ws + bp.stats_bytes);
  float** mats[] = {&x.Am, &x.Um, &x.Xm, &x.Sst, &x.Rin};
  for (int i = 0; i < 5; ++i) *mats[i] = reinterpret_cast<float*>(ws + bp.mat_off + i * bp.mat_bytes);
  x.slots = reinterpret_cast<float*>(ws + bp.slot_off);
  x.n_slots = bp.n_slots;
  x.slot_floats = bp.slot_floats;
  x.dw_part = reinterpret_cast<float*>(ws + bp.part_off);
  x.dw_slices = kDwSlices;
  x.C = cfg->gdn_chunk;
  x.scale = plan.scale;
  x.attn_mfma = plan.attn == Impl::Mfma && cfg->out_dtype == HLTA_BF16;
  if (lse && x.attn_mfma) {
    x.lse2 = const_cast<float*>(lse);   // read only: the statistics kernel is skipped
    x.lse_given = 1;
  }
  hipError_t e = launch_bwd(x, cfg->d, cfg->in_dtype, cfg->out_dtype, st);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return HLTA_OK;
}

extern "C" {

hlta_status hlta_bwd(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                     const float* b, const float* mix_w, const float* S0, const void* o_swa, const void* o_dswa,
                     const void* o_gdn, const void* d_mix, float* dq, float* dk, float* dv, float* da, float* db,
                     float* dmix_w, float* dS0, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  return bwd_impl(cfg, q, k, v, a, b, mix_w, S0, o_swa, o_dswa, o_gdn, d_mix, dq, dk, dv, da, db, dmix_w, dS0,
                  nullptr, workspace, ws_bytes, stream);
}

hlta_status hlta_bwd_lse(const hlta_config* cfg, const void* q, const void* k, const void* v, const float* a,
                         const float* b, const float* mix_w, const float* S0, const void* o_swa, const void* o_dswa,
                         const void* o_gdn, const void* d_mix, const float* lse, float* dq, float* dk, float* dv,
                         float* da, float* db, float* dmix_w, float* dS0, void* workspace, size_t ws_bytes,
                         void* stream) {
  clear_error();
  if (cfg && int64_t(cfg->T) * cfg->P > 0) HLTA_TRY(need(lse, "lse"));
  return bwd_impl(cfg, q, k, v, a, b, mix_w, S0, o_swa, o_dswa, o_gdn, d_mix, dq, dk, dv, da, db, dmix_w, dS0,
                  lse, workspace, ws_bytes, stream);
}

static hlta_status check_stream(const hlta_config* cfg, const hlta_stream_state* st) {
  if (!st) return fail(HLTA_E_NULL, "stream state is NULL");
  HLTA_TRY(need(st->S, "state S"));
  HLTA_TRY(need(st->ring_k, "ring_k"));
  HLTA_TRY(need(st->ring_v, "ring_v"));
  const long long need_frames = cfg->swa_frames - 1 > (long long)cfg->dswa_dilation * cfg->dswa_taps
                                    ? cfg->swa_frames - 1
                                    : (long long)cfg->dswa_dilation * cfg->dswa_taps;
  if (st->ring_frames < 1 || st->ring_frames < need_frames)
    return fail(HLTA_E_STATE, "ring_frames must be >= max(1, W-1, dil*taps) = " +
                                  std::to_string(need_frames < 1 ? 1 : need_frames));
  if (st->frames_done < 0) return fail(HLTA_E_STATE, "frames_done is negative");
  return HLTA_OK;
}

hlta_status hlta_stream_load_prefix(const hlta_config* cfg, hlta_stream_state* st, const void* k_prefix,
                                    const void* v_prefix, int32_t prefix_frames, const float* S_prefix,
                                    void* stream) {
  clear_error();
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(check_stream(cfg, st));
  if (prefix_frames < 0) return fail(HLTA_E_SHAPE, "prefix_frames must be >= 0");
  if (prefix_frames > 0) {
    HLTA_TRY(need(k_prefix, "k_prefix"));
    HLTA_TRY(need(v_prefix, "v_prefix"));
  }
  HLTA_TRY(maybe(S_prefix, "S_prefix"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long keep = prefix_frames < st->ring_frames ? prefix_frames : st->ring_frames;
  const long long first = prefix_frames - keep;
  const long long frame_elems = (long long)cfg->P * cfg->H * cfg->d;
  const int elem = int(dtype_bytes(cfg->in_dtype));
  hipError_t e = launch_ring_store(k_prefix, prefix_frames, 0, st->ring_k, st->ring_frames, first, keep, cfg->B,
                                   frame_elems, elem, s);
  if (e == hipSuccess)
    e = launch_ring_store(v_prefix, prefix_frames, 0, st->ring_v, st->ring_frames, first, keep, cfg->B,
                          frame_elems, elem, s);
  if (e == hipSuccess && cfg->rope_theta > 0.f && keep > 0)
    e = launch_rope_ring(st->ring_k, cfg->B, st->ring_frames, first, int(keep), cfg->H, cfg->d, cfg->P,
                         cfg->rope_grid_w, cfg->rope_theta, cfg->in_dtype, s);
  if (e != hipSuccess) return hip_fail(e, "ring store");
  e = S_prefix == st->S ? hipSuccess : launch_copy_or_zero(st->S, S_prefix, state_bytes(cfg), s);
  if (e != hipSuccess) return hip_fail(e, "state copy");
  st->frames_done = prefix_frames;
  return HLTA_OK;
}

// One streaming step. frames == null: every rollout appends frame
// st->frames_done. Otherwise rollout b appends frame frames[b], or sits the
// step out when frames[b] == -1.
static hlta_status step_frame_impl(const hlta_config* cfg, hlta_stream_state* st, int64_t* frames, const void* q_f,
                                   const void* k_f, const void* v_f, const float* a_f, const float* b_f,
                                   const float* mix_w, void* o_swa, void* o_dswa, void* o_gdn, void* o_mix,
                                   int32_t commit, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  HLTA_TRY(check_config(cfg));
  HLTA_TRY(check_stream(cfg, st));
  Plan plan;
  HLTA_TRY(make_plan(cfg, cfg->P, &plan));
  HLTA_TRY(need(q_f, "q_f"));
  HLTA_TRY(need(k_f, "k_f"));
  HLTA_TRY(need(v_f, "v_f"));
  HLTA_TRY(check_outputs(a_f, b_f, mix_w, o_swa, o_dswa, o_gdn, o_mix));
  HLTA_TRY(check_workspace(plan, workspace, ws_bytes));
  AttnParams at{};
  unsigned long long skip = 0;
  if (frames) {
    if (cfg->B > kMaxRollouts)
      return fail(HLTA_E_UNSUPPORTED, "per-rollout positions support at most " + std::to_string(kMaxRollouts) +
                                          " rollouts (B = " + std::to_string(cfg->B) + ")");
    int active = 0;
    for (int b = 0; b < cfg->B; ++b) {
      if (frames[b] < -1)
        return fail(HLTA_E_STATE, "frames[" + std::to_string(b) + "] = " + std::to_string(frames[b]) +
                                      " (a frame index, or -1 to leave the rollout out)");
      if (frames[b] == -1) skip |= 1ull << b;
      else ++active;
      at.ro.frame[b] = frames[b] < 0 ? 0 : frames[b];
    }
    if (active == 0) return HLTA_OK;
    at.per_rollout = 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long long f = st->frames_done;
  at.q = q_f;
  at.k = k_f;
  at.v = v_f;
  at.ring_k = st->ring_k;
  at.ring_v = st->ring_v;
  at.o_swa = o_swa;
  at.o_dswa = o_dswa;
  at.B = cfg->B;
  at.H = cfg->H;
  at.T = 1;
  at.P = cfg->P;
  at.W = cfg->swa_frames;
  at.dil = cfg->dswa_dilation;
  at.taps = cfg->dswa_taps;
  at.R = st->ring_frames;
  at.f0 = f;
  at.ro.skip = skip;
  HLTA_TRY(run_layer(cfg, plan, q_f, k_f, v_f, a_f, b_f, st->S, commit ? st->S : nullptr, o_gdn, mix_w, o_mix,
                     workspace, at, s));
  if (commit) {
    const long long frame_elems = (long long)cfg->P * cfg->H * cfg->d;
    const int elem = int(dtype_bytes(cfg->in_dtype));
    hipError_t e = hipSuccess;
    // the ring keeps the keys the attention read (rotated when the rotary embedding is on)
    if (!frames) {
      e = launch_ring_store(at.k, 1, f, st->ring_k, st->ring_frames, f, 1, cfg->B, frame_elems, elem, s);
      if (e == hipSuccess)
        e = launch_ring_store(v_f, 1, f, st->ring_v, st->ring_frames, f, 1, cfg->B, frame_elems, elem, s);
    } else {
      // each rollout that stepped into the slot of its own frame
      e = launch_ring_store_rollouts(at.k, st->ring_k, st->ring_frames, cfg->B, frame_elems, elem, at.ro, s);
      if (e == hipSuccess)
        e = launch_ring_store_rollouts(v_f, st->ring_v, st->ring_frames, cfg->B, frame_elems, elem, at.ro, s);
    }
    if (e != hipSuccess) return hip_fail(e, "ring store");
    if (!frames) st->frames_done = f + 1;
    else
      for (int b = 0; b < cfg->B; ++b)
        if (frames[b] >= 0) ++frames[b];
  }
  return HLTA_OK;
}

hlta_status hlta_step_frame(const hlta_config* cfg, hlta_stream_state* st, const void* q_f, const void* k_f,
                            const void* v_f, const float* a_f, const float* b_f, const float* mix_w, void* o_swa,
                            void* o_dswa, void* o_gdn, void* o_mix, int32_t commit, void* workspace,
                            size_t ws_bytes, void* stream) {
  return step_frame_impl(cfg, st, nullptr, q_f, k_f, v_f, a_f, b_f, mix_w, o_swa, o_dswa, o_gdn, o_mix, commit,
                         workspace, ws_bytes, stream);
}

hlta_status hlta_step_frame_rollouts(const hlta_config* cfg, hlta_stream_state* st, int64_t* frames,
                                     const void* q_f, const void* k_f, const void* v_f, const float* a_f,
                                     const float* b_f, const float* mix_w, void* o_swa, void* o_dswa, void* o_gdn,
                                     void* o_mix, int32_t commit, void* workspace, size_t ws_bytes,
                                     void* stream) {
  if (!frames) {
    clear_error();
    return fail(HLTA_E_NULL, "frames is NULL");
  }
  return step_frame_impl(cfg, st, frames, q_f, k_f, v_f, a_f, b_f, mix_w, o_swa, o_dswa, o_gdn, o_mix, commit,
                         workspace, ws_bytes, stream);
}

hlta_status hlta_ceiling_mfma_bf16(float* sink, uint64_t* clocks, int32_t workgroups, int32_t iters, void* stream) {
  clear_error();
  HLTA_TRY(need(sink, "sink"));
  HLTA_TRY(maybe(clocks, "clocks"));
  if (workgroups < 1 || iters < 1) return fail(HLTA_E_SHAPE, "workgroups and iters must be >= 1");
  const hipError_t e = launch_ceiling_mfma(sink, reinterpret_cast<unsigned long long*>(clocks), workgroups, iters,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "MFMA ceiling launch");
  return HLTA_OK;
}

hlta_status hlta_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream) {
  clear_error();
  HLTA_TRY(need(src, "src"));
  HLTA_TRY(need(dst, "dst"));
  if (bytes % 16 != 0) return fail(HLTA_E_SHAPE, "bytes must be a multiple of 16");
  const hipError_t e = launch_ceiling_copy(src, dst, bytes, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy ceiling launch");
  return HLTA_OK;
}

}  // extern "C"
