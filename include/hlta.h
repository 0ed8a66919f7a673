/*
 * hlta.h - C ABI of the MI355X (gfx950) Hybrid Linear Temporal Attention library.
 *
 * HLTA (Kairos abstract on chatpaper.ai, point (2); Kairos summary page on
 * researchpapers.dev, section on how the hybrid linear temporal attention limits
 * drift) mixes three temporal branches over latent-video tokens:
 *   - SWA:  sliding-window softmax attention over whole latent frames (local dynamics);
 *   - DSWA: softmax attention over dilated past frames (mid-range dependencies);
 *   - GDN:  gated linear attention with the delta update rule, a fixed-size
 *           state S per head that is the persistent global memory
 *           (Kairos related-work page, row A; long-context page, section 06):
 *             S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t.
 * Each call returns the three branch outputs separately and their weighted sum.
 *
 * Conventions shared by every entry point
 *   Layout.   Tokens are frame-major: token t = f*P + p of latent frame f.
 *             q, k, v, outputs: [B, L, H, d] row-major (heads interleaved per
 *             token, as a fused QKV projection emits them), L = T*P.
 *             a, b (gates): [B, L, H] float32. mix_w: [H, 3] float32
 *             (weights of SWA, DSWA, GDN). States S: [B, H, d, d] float32,
 *             S[b][h][i][j] = row i (value dim) , column j (key dim).
 *   Memory.   Every pointer is a device pointer owned by the caller, 16-byte
 *             aligned. The library allocates nothing and keeps no per-call
 *             state; scratch memory is the caller's workspace.
 *   Streams.  `stream` is a hipStream_t (NULL = the default stream). Work is
 *             enqueued asynchronously; outputs are valid after the caller
 *             synchronises the stream. Calls on one stream run in order.
 *   Errors.   Arguments are validated on the host before anything is launched;
 *             a failed check returns a non-zero hlta_status, launches nothing
 *             and leaves a message in hlta_last_error(). A launch failure
 *             returns HLTA_E_HIP. Faults inside kernels surface at the caller's
 *             synchronisation. Gate values are not checked: a in (0, 1] and
 *             b in [0, 1] give the contractive memory; a = 0 is accepted (its
 *             logarithm is floored at -80). With cfg->gate_logits = 1 they
 *             are logits instead (below).
 */
#ifndef HLTA_H
#define HLTA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HLTA_ABI_VERSION 2

typedef enum {
  HLTA_OK = 0,
  HLTA_E_NULL = 1,        /* a required pointer is NULL */
  HLTA_E_SHAPE = 2,       /* a size is out of range */
  HLTA_E_DTYPE = 3,       /* unsupported dtype pair */
  HLTA_E_UNSUPPORTED = 4, /* valid but not implemented (e.g. d = 96) */
  HLTA_E_WORKSPACE = 5,   /* workspace NULL or smaller than required */
  HLTA_E_ALIGN = 6,       /* a pointer is not 16-byte aligned */
  HLTA_E_STATE = 7,       /* streaming state inconsistent with the config */
  HLTA_E_HIP = 8          /* a HIP runtime call or launch failed */
} hlta_status;

typedef enum { HLTA_F32 = 0, HLTA_BF16 = 1 } hlta_dtype;

typedef enum {
  HLTA_IMPL_AUTO = 0,     /* MFMA kernels where the shape has them, else generic */
  HLTA_IMPL_GENERIC = 1,  /* plain fp32-arithmetic kernels, any supported shape */
  HLTA_IMPL_MFMA = 2      /* bf16 MFMA kernels; HLTA_E_UNSUPPORTED where absent */
} hlta_impl;

/* Sizes and options of one HLTA layer. */
typedef struct {
  int32_t B;              /* batch (independent clips or rollouts), >= 1 */
  int32_t H;              /* heads, >= 1 */
  int32_t T;              /* latent frames, >= 0 (0 = empty call, returns HLTA_OK) */
  int32_t P;              /* tokens per latent frame, >= 1 */
  int32_t d;              /* head dim, d_k = d_v = d, one of 32, 64, 128 */
  int32_t swa_frames;     /* W >= 0: SWA reads frames f-W+1 .. f (W counts the current frame) */
  int32_t dswa_dilation;  /* dil >= 1 */
  int32_t dswa_taps;      /* taps >= 0: DSWA reads frames f - dil*r, r = 1..taps */
  int32_t gdn_chunk;      /* C: chunk length of the chunked delta rule, 16, 32 or 64 */
  float softmax_scale;    /* logit scale; <= 0 selects 1/sqrt(d) */
  int32_t gdn_l2norm_qk;  /* 1: GDN L2-normalises q and k per token (eps 1e-6 in the sqrt) */
  int32_t in_dtype;       /* hlta_dtype of q, k, v and of the ring buffers */
  int32_t out_dtype;      /* hlta_dtype of every output: (f32,f32), (bf16,bf16), (bf16,f32) */
  int32_t impl;           /* hlta_impl */
  float rope_theta;       /* > 0: rotary embedding of the softmax branches' q and k (below); 0: none */
  int32_t rope_grid_h;    /* with rope_theta > 0: the token grid of a latent frame, */
  int32_t rope_grid_w;    /*   rope_grid_h * rope_grid_w == P, token p at (p / grid_w, p % grid_w) */
  int32_t gate_logits;    /* 1: a and b hold logits; the memory uses sigmoid(a) and sigmoid(b) (below) */
} hlta_config;

/*
 * Rotary embedding of the softmax branches (optional, rope_theta > 0). The
 * pages give the local branches as windows over latent frames and name no
 * positional scheme; the reading implemented: a token's position is
 * (absolute latent frame, row, column); its d/2 coordinate pairs
 * (x[2i], x[2i+1]) are rotated as complex numbers by pos_axis * theta^(-j/n),
 * the first d/8 pairs by the frame, the next half of the rest by the row, the
 * others by the column (j = the pair's index within its axis, n = the axis's
 * pair count). q and k of SWA and DSWA are rotated (rounded once to
 * in_dtype); the memory branch reads them unrotated. Streaming rings hold
 * rotated keys. hlta_fwd and the streaming calls support it (its rotated
 * copies live in the workspace); hlta_attn_fwd, which has no workspace,
 * returns HLTA_E_UNSUPPORTED for it.
 *
 * Gate logits (optional, gate_logits = 1). The pages give the decay and write
 * gates but not how a layer produces them; the reading implemented: a and b
 * arrive as raw per-token logits and the memory branch applies the logistic
 * function as it loads them (in fp32: log a = log sigmoid(x_a), computed
 * without cancellation, floored at -80; b = sigmoid(x_b)). Both gates then lie
 * in (0, 1), the contractive range.
 */

/* ABI version of the loaded library (HLTA_ABI_VERSION). */
int32_t hlta_abi_version(void);

/* Static string for a status code. */
const char* hlta_status_string(int32_t status);

/* Detail of the last failed call on this thread ("" if none). */
const char* hlta_last_error(void);

/* Host-only check of a config (no GPU needed). */
hlta_status hlta_validate_config(const hlta_config* cfg);

/* Bytes of device workspace hlta_fwd needs for cfg (0 on an invalid config). */
size_t hlta_fwd_workspace_bytes(const hlta_config* cfg);

/*
 * hlta_fwd - HLTA forward over whole clips.
 *
 * Per batch row b, head h and latent frame f:
 *   o_swa  = softmax attention of the queries of frame f over every key of
 *            frames max(0, f-W+1) .. f (bidirectional inside a frame, causal
 *            across frames), logits scaled by softmax_scale;
 *   o_dswa = the same over frames f - dil*r, r = 1..taps, f - dil*r >= 0;
 *            rows of a frame with no such frame are 0;
 *   o_gdn  = the gated delta rule run over the tokens in order from S0
 *            (computed in chunks of C tokens; equal to the token recurrence);
 *   o_mix  = w[h,0]*o_swa + w[h,1]*o_dswa + w[h,2]*o_gdn, evaluated in fp32
 *            from the three outputs as stored, rounded once to out_dtype.
 * The memory and its contraction: Kairos related-work page (row A, and the
 * delta section on contraction rho < 1); long-context page, section 06.
 *
 * q, k, v   [B, L, H, d] in_dtype (read only)
 * a, b      [B, L, H] float32 decay and write gates (read only)
 * mix_w     [H, 3] float32 (read only)
 * S0        [B, H, d, d] float32 start state, or NULL for zero
 * o_swa, o_dswa, o_gdn, o_mix   [B, L, H, d] out_dtype (written; no aliasing)
 * S_out     [B, H, d, d] float32 final state, or NULL; may equal S0
 * workspace device buffer of at least hlta_fwd_workspace_bytes(cfg) bytes
 */
hlta_status hlta_fwd(const hlta_config* cfg,
                     const void* q, const void* k, const void* v,
                     const float* a, const float* b, const float* mix_w,
                     const float* S0,
                     void* o_swa, void* o_dswa, void* o_gdn, void* o_mix,
                     float* S_out,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * hlta_fwd_noalloc - hlta_fwd without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. It calls no allocating routine; its
 * scratch is a fixed device array of HLTA_NOALLOC_SCRATCH_BYTES per GPU,
 * reserved when the library's code is loaded on that GPU and held until the
 * process ends. Results equal hlta_fwd's bit for bit (the same kernels).
 *
 * A call whose hlta_fwd_workspace_bytes(cfg) exceeds the array returns
 * HLTA_E_WORKSPACE before anything is launched. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (different streams, or
 * different host threads) race on it and must be ordered by the caller. The
 * array keeps the last call's contents; a call reads only scratch it has
 * written itself. The stream must belong to the current device. Other
 * arguments and errors as in hlta_fwd.
 */
#define HLTA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hlta_status hlta_fwd_noalloc(const hlta_config* cfg,
                             const void* q, const void* k, const void* v,
                             const float* a, const float* b, const float* mix_w,
                             const float* S0,
                             void* o_swa, void* o_dswa, void* o_gdn, void* o_mix,
                             float* S_out, void* stream);

/*
 * hlta_gdn_fwd - the memory branch alone: o_gdn and S_out exactly as hlta_fwd
 * computes them (the gated delta rule of the Kairos related-work page, row A,
 * and of the long-context page, section 06). Arguments as in hlta_fwd.
 */
hlta_status hlta_gdn_fwd(const hlta_config* cfg,
                         const void* q, const void* k, const void* v,
                         const float* a, const float* b, const float* S0,
                         void* o_gdn, float* S_out,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * hlta_attn_fwd - the two softmax branches (Kairos abstract, point (2):
 * sliding windows for local dynamics, dilated windows for mid-range
 * dependencies) and the mix, exactly as hlta_fwd computes them. o_gdn is read
 * by the mix (it is the output of a previous hlta_gdn_fwd on the same
 * stream); hlta_gdn_fwd followed by hlta_attn_fwd equals hlta_fwd. Needs no
 * workspace. Arguments as in hlta_fwd.
 */
hlta_status hlta_attn_fwd(const hlta_config* cfg,
                          const void* q, const void* k, const void* v,
                          const float* mix_w, const void* o_gdn,
                          void* o_swa, void* o_dswa, void* o_mix, void* stream);

/*
 * The other split of hlta_fwd, in its own order: hlta_attn_branches followed
 * by hlta_gdn_mix_fwd on one stream equals hlta_fwd bit for bit, and equals
 * hlta_gdn_fwd followed by hlta_attn_fwd.
 *
 * hlta_attn_branches - the two softmax branches alone (Kairos abstract,
 * point (2)): o_swa and o_dswa. Needs no workspace; HLTA_E_UNSUPPORTED with
 * the rotary embedding on. Arguments as in hlta_fwd.
 */
hlta_status hlta_attn_branches(const hlta_config* cfg,
                               const void* q, const void* k, const void* v,
                               void* o_swa, void* o_dswa, void* stream);

/*
 * hlta_gdn_mix_fwd - the memory branch (Kairos related-work page, row A;
 * long-context page, section 06) and the mix (Kairos page, HLTA section):
 * o_gdn, S_out and o_mix = w_swa o_swa + w_dswa o_dswa + w_gdn o_gdn per
 * head, from the o_swa, o_dswa given (read only, as stored by a previous
 * hlta_attn_branches on the same stream). Arguments and errors as in
 * hlta_fwd.
 */
hlta_status hlta_gdn_mix_fwd(const hlta_config* cfg,
                             const void* q, const void* k, const void* v,
                             const float* a, const float* b, const float* mix_w,
                             const float* S0, const void* o_swa, const void* o_dswa,
                             void* o_gdn, void* o_mix, float* S_out,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * hlta_attn_fwd_lse - hlta_attn_fwd that also writes the softmax row
 * statistics the backward needs (each query row's log-sum-exp, which the
 * tiled exact attention of the long-context page, section 03, carries
 * anyway), so that hlta_bwd_lse does not recompute them:
 * lse  [2, B, H, L] float32 (branch SWA then DSWA, batch row, head, token):
 *      log2 of the row's softmax denominator with scores in log2 units,
 *      log2 sum_j exp(scale * q . k_j); 0 for a row whose branch has no key
 *      (written; the caller owns it).
 * Outputs o_swa, o_dswa, o_mix are bit for bit those of hlta_attn_fwd. Other
 * arguments and errors as hlta_attn_fwd; lse NULL gives HLTA_E_NULL.
 */
hlta_status hlta_attn_fwd_lse(const hlta_config* cfg,
                              const void* q, const void* k, const void* v,
                              const float* mix_w, const void* o_gdn,
                              void* o_swa, void* o_dswa, void* o_mix,
                              float* lse, void* stream);

/*
 * FP8 variant of the softmax branches. The pages mention low-precision
 * attention without a method; the variant implemented quantises q, k, v per
 * (batch row, head) to e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite value 448) and runs SWA and DSWA with 8-bit MFMA
 * products accumulated in fp32, the softmax in fp32 and P rounded to e4m3.
 *
 * hlta_quantize_fp8 - codes and scales: for each (b, h) and tensor,
 * s = max|x| / 448 (1 when the head is all zero), code = e4m3(x / s) with x / s
 * in float32 clamped to +-448, rounded to nearest, ties to even.
 * q, k, v [B, L, H, d] in_dtype (read only); q8, k8, v8 [B, L, H, d] bytes
 * (written); scales [B, H, 3] float32 (written; s of q, k, v).
 */
hlta_status hlta_quantize_fp8(const hlta_config* cfg, const void* q, const void* k, const void* v,
                              void* q8, void* k8, void* v8, float* scales, void* stream);

/*
 * hlta_attn_fwd_fp8 - hlta_attn_fwd on e4m3 codes: o_swa, o_dswa equal exact
 * softmax attention over the dequantised inputs (code x scale) up to the
 * rounding of P to e4m3 (numerator and denominator both use the rounded P);
 * o_mix as in hlta_attn_fwd. d = 128 and P >= 64 (HLTA_E_UNSUPPORTED
 * otherwise); cfg->in_dtype is not used; no rotary embedding (rotate before
 * quantising). Arguments as in hlta_attn_fwd with q8, k8, v8, scales as
 * hlta_quantize_fp8 writes them.
 */
hlta_status hlta_attn_fwd_fp8(const hlta_config* cfg, const void* q8, const void* k8, const void* v8,
                              const float* scales, const float* mix_w, const void* o_gdn,
                              void* o_swa, void* o_dswa, void* o_mix, void* stream);

/*
 * hlta_bwd - gradients of the operator for training: with L = <d_mix, o_mix>,
 * the branch gradients are do_i = w[h,i] * d_mix (the mix is linear) and
 *   dmix_w[h,i] = <d_mix, o_i> over the stored branch outputs;
 *   softmax branches: the exact gradient of softmax attention over each query
 *     frame's key set (the branches are exact attention: long-context page,
 *     section 03), recomputed from q, k, v with per-row log-sum-exp;
 *   memory: the exact gradient of the gated delta rule of hlta_fwd (Kairos
 *     related-work page, row A; long-context page, section 06): per chunk its
 *     transition, own state and own adjoint, chains over chunks for every
 *     chunk's start state and incoming adjoint, then each chunk's token
 *     gradients in the chunk's matrix (UT / WY) form; through the L2
 *     normalisation of q and k when on.
 * dq, dk, dv receive the sum over the three branches.
 *
 * q, k, v, a, b, mix_w, S0   the forward's inputs (read only)
 * o_swa, o_dswa, o_gdn       the forward's branch outputs, out_dtype (read only)
 * d_mix      [B, L, H, d] out_dtype, dL/do_mix (read only)
 * dq, dk, dv [B, L, H, d] float32 (written)
 * da, db     [B, L, H] float32, gradients of the gates a and b (written)
 * dmix_w     [H, 3] float32 (written)
 * dS0        [B, H, d, d] float32 gradient of the start state, or NULL
 * workspace  device buffer of at least hlta_bwd_workspace_bytes(cfg) bytes
 *            (per chunk of gdn_chunk tokens of each batch row and head: five
 *            d x d fp32 matrices and the chunk's own 64-row matrices, about
 *            0.94 MB at d = 128; plus the softmax statistics)
 * The gates are taken as given (gate_logits = 1 and the rotary embedding give
 * HLTA_E_UNSUPPORTED). The memory's gradients are evaluated with fp32
 * accumulation, their matrix products on bf16 MFMA with each fp32 factor split
 * into two bf16 parts (close to fp32 accuracy). The softmax branches' are in
 * fp32, except with bf16 inputs and outputs, d = 128 and
 * P >= 64, where they run on bf16 MFMA (fp32 accumulation; P and dS rounded
 * to bf16 for their products; D = do . o from the stored outputs).
 * Validation (NULL, alignment, workspace size, config) happens before any
 * launch; outputs must not alias inputs; results are deterministic (no
 * atomics). Work is enqueued on `stream`; nothing is allocated.
 */
size_t hlta_bwd_workspace_bytes(const hlta_config* cfg);
hlta_status hlta_bwd(const hlta_config* cfg,
                     const void* q, const void* k, const void* v,
                     const float* a, const float* b, const float* mix_w, const float* S0,
                     const void* o_swa, const void* o_dswa, const void* o_gdn, const void* d_mix,
                     float* dq, float* dk, float* dv, float* da, float* db,
                     float* dmix_w, float* dS0,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * hlta_bwd_lse - hlta_bwd with the softmax row statistics given: lse as
 * hlta_attn_fwd_lse wrote it for the same cfg, q and k (read only). Where the
 * softmax branches run on bf16 MFMA (see above) their statistics pass is
 * skipped; elsewhere the statistics are recomputed and lse is not read. Other
 * arguments, results and errors as hlta_bwd (same workspace size); lse NULL
 * with L > 0 gives HLTA_E_NULL.
 */
hlta_status hlta_bwd_lse(const hlta_config* cfg,
                         const void* q, const void* k, const void* v,
                         const float* a, const float* b, const float* mix_w, const float* S0,
                         const void* o_swa, const void* o_dswa, const void* o_gdn, const void* d_mix,
                         const float* lse,
                         float* dq, float* dk, float* dv, float* da, float* db,
                         float* dmix_w, float* dS0,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Streaming (Kairos article on zhichai.net, section 2.3: streaming tokens so
 * generation proceeds incrementally without recomputing the sequence).
 *
 * A stream holds, per rollout b: the GDN state S [B, H, d, d] float32 and a
 * ring of the K and V of the last ring_frames frames, [B, R, P, H, d]
 * in_dtype each; frame j lives in slot j mod R. frames_done counts the frames
 * appended so far (all B rollouts advance together). The caller allocates the
 * three buffers (hlta_stream_ring_bytes gives the size of each ring) and owns
 * the struct; saving and restoring (S, rings, frames_done) resumes a stream.
 * R must be at least max(W - 1, dil * taps) so that every frame a step reads
 * is still in the ring. cfg->T is ignored by the streaming calls.
 */
typedef struct {
  float* S;               /* [B, H, d, d] float32 */
  void* ring_k;           /* [B, R, P, H, d] in_dtype */
  void* ring_v;           /* [B, R, P, H, d] in_dtype */
  int32_t ring_frames;    /* R */
  int64_t frames_done;    /* frames appended so far */
} hlta_stream_state;

/* Bytes of one ring buffer (K or V) for R frames (0 on an invalid config). */
size_t hlta_stream_ring_bytes(const hlta_config* cfg, int32_t ring_frames);

/*
 * Start a stream from a prefix of prefix_frames frames: copies the K and V of
 * the last min(prefix_frames, R) prefix frames into their ring slots, copies
 * S_prefix (or zeros when NULL) into st->S and sets frames_done = prefix_frames.
 * k_prefix, v_prefix: [B, prefix_frames*P, H, d] in_dtype (may be NULL only
 * when prefix_frames == 0). S_prefix is typically the S_out of hlta_fwd over
 * the prefix.
 */
hlta_status hlta_stream_load_prefix(const hlta_config* cfg, hlta_stream_state* st,
                                    const void* k_prefix, const void* v_prefix,
                                    int32_t prefix_frames, const float* S_prefix,
                                    void* stream);

/* Bytes of device workspace hlta_step_frame needs (0 on an invalid config). */
size_t hlta_step_workspace_bytes(const hlta_config* cfg);

/*
 * hlta_step_frame - append frame f = st->frames_done to every rollout.
 *
 * Outputs equal rows [f*P, (f+1)*P) of hlta_fwd over frames 0..f of the same
 * rollout: SWA reads frames f-W+1 .. f-1 from the ring and frame f from the
 * inputs; DSWA reads frames f - dil*r from the ring; GDN runs the frame's P
 * tokens from st->S. With commit != 0 the call then updates st->S in place,
 * writes k_f, v_f to ring slot f mod R and increments st->frames_done; with
 * commit == 0 the stream is left unchanged (several evaluations of one frame).
 *
 * q_f, k_f, v_f [B, P, H, d] in_dtype; a_f, b_f [B, P, H] float32;
 * mix_w [H, 3]; o_* [B, P, H, d] out_dtype.
 */
hlta_status hlta_step_frame(const hlta_config* cfg, hlta_stream_state* st,
                            const void* q_f, const void* k_f, const void* v_f,
                            const float* a_f, const float* b_f, const float* mix_w,
                            void* o_swa, void* o_dswa, void* o_gdn, void* o_mix,
                            int32_t commit, void* workspace, size_t ws_bytes, void* stream);

/*
 * hlta_step_frame_rollouts - one streaming step in which every rollout is at
 * its own position (rollouts started at different times, or advanced by
 * different numbers of steps, e.g. several streams served together). The
 * per-rollout counts live in frames, a host array of B entries owned by the
 * caller (st->frames_done is not used): rollout b appends frame frames[b],
 * which must equal the number of frames it has appended so far, or sits the
 * step out when frames[b] == -1 (its output rows are not written and its
 * state, ring slots and count stay as they are). Outputs of a stepping
 * rollout equal those of hlta_step_frame on a stream holding that rollout
 * alone. With commit != 0 each stepping rollout's S and ring slot
 * frames[b] mod R are updated and frames[b] is incremented.
 * B <= 64 (HLTA_E_UNSUPPORTED otherwise); an entry below -1 is HLTA_E_STATE,
 * frames == NULL is HLTA_E_NULL. Other arguments as in hlta_step_frame; rows
 * of q_f .. b_f belonging to rollouts that sit out are not read.
 */
hlta_status hlta_step_frame_rollouts(const hlta_config* cfg, hlta_stream_state* st, int64_t* frames,
                                     const void* q_f, const void* k_f, const void* v_f,
                                     const float* a_f, const float* b_f, const float* mix_w,
                                     void* o_swa, void* o_dswa, void* o_gdn, void* o_mix,
                                     int32_t commit, void* workspace, size_t ws_bytes, void* stream);

/*
 * Measured ceilings (not part of the operator): microbenchmarks of the GPU the
 * library runs on, so that a kernel's roofline fraction can be stated against
 * what the chip sustains beside its published peak. The caller times them
 * (e.g. with events on `stream`).
 *
 * hlta_ceiling_mfma_bf16 - dense bf16 matrix-core loop: `workgroups`
 * workgroups of 4 waves; every wave issues iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (32 x 32 x 16 x 2 = 32768 flop
 * each), so one call performs workgroups * 4 * iters * 8 * 32768 flop.
 * sink: device float[workgroups * 256], written (keeps the products live).
 * clocks: device uint64[2] or NULL: core-clock ticks and 100 MHz
 * reference-clock ticks that workgroup 0 spent in its loop (their ratio times
 * 100 MHz is the clock the chip held). workgroups, iters >= 1, else
 * HLTA_E_SHAPE; sink NULL is HLTA_E_NULL; pointers must be 16-byte aligned.
 */
hlta_status hlta_ceiling_mfma_bf16(float* sink, uint64_t* clocks, int32_t workgroups, int32_t iters,
                                   void* stream);

/*
 * hlta_ceiling_copy - HBM streaming copy: dst[0 .. bytes) = src[0 .. bytes)
 * with 16-byte loads and stores (2 * bytes of traffic per call). Device
 * buffers, 16-byte aligned, not overlapping; bytes a multiple of 16, else
 * HLTA_E_SHAPE.
 */
hlta_status hlta_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HLTA_H */
