"""Float64 CPU oracle of Hybrid Linear Temporal Attention (HLTA).

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module. The GPU library never
calls it and shares no code with it; the only common module is the seeded
input generator (hybrid_linear_temporal_amd/inputs.py).

Plain and slow on purpose: every function is the plain definition of what it
computes, in float64, one (batch, head) at a time.

What HLTA is (Kairos abstract on chatpaper.ai, point (2); Kairos summary page
on researchpapers.dev, section on how the hybrid linear temporal attention
limits drift): three temporal branches over latent-video tokens, namely
sliding-window softmax attention for local dynamics, dilated sliding windows for
mid-range dependencies, and gated linear attention with a delta update rule as
the persistent global memory.

Readings taken where the pages are silent:
  * tokens are frame-major, t = f*P + p; frame(t) = t // P;
  * the softmax branches are frame-block causal: a query of frame f sees every
    token of each frame in its frame set, bidirectional inside a frame;
  * SWA frame set {f - j : 0 <= j < W}: W counts the current frame;
  * DSWA frame set {f - dil*r : 1 <= r <= taps}; frames below 0 are skipped;
    a query with an empty frame set outputs zeros;
  * softmax scale 1/sqrt(d) unless given; no bias; no positional term unless
    the optional rotary embedding of the softmax branches is asked for (its
    variant is not on the pages; the reading is stated at `rope`);
  * the memory follows the gated delta rule, one token at a time in token order
    (raster inside a frame), with per-token per-head gates a (decay) and b
    (write strength) used as given, in-op L2 normalisation of q and k with
    eps = 1e-6 inside the square root, and the read o_t = S_t q_t taken after
    the token's own update;
  * the three outputs are combined as o_mix = w0*o_swa + w1*o_dswa + w2*o_gdn
    with caller weights w[h, :] and nothing else;
  * optionally the gates arrive as logits and the memory uses their logistic
    function (the pages give no gate parameterization; see `gates_from_logits`).
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

L2_EPS = 1e-6
LOG_A_FLOOR = -80.0   # log of the decay gate is floored here (a = 0 stays finite)


# ---------------------------------------------------------------------------
# token / frame indexing
# ---------------------------------------------------------------------------

def swa_frames(f: int, W: int) -> list[int]:
    """Frames a query frame f reads in the sliding-window branch: the current
    frame and the W-1 before it (Kairos abstract, point (2): sliding-window
    attention for local dynamics)."""
    return [f - j for j in range(W) if f - j >= 0]


def dswa_frames(f: int, dil: int, taps: int) -> list[int]:
    """Frames a query frame f reads in the dilated branch: f - dil*r for
    r = 1..taps (Kairos abstract, point (2): dilated sliding windows for
    mid-range dependencies)."""
    return [f - dil * r for r in range(1, taps + 1) if f - dil * r >= 0]


# ---------------------------------------------------------------------------
# softmax branches
# ---------------------------------------------------------------------------

def frame_softmax_attention(q, k, v, T, P, frames_of, scale=None):
    """Exact softmax attention of each query frame over the keys of its frame set.

    q, k, v: [T*P, d] float64 of one (batch, head). frames_of(f) -> list of key
    frames. Every legal (query, key) pair is used, as exact attention does
    (long-context page, section 03 on FlashAttention: tiling changes memory
    traffic, not the set of pairs or the result). Rows with no key frame are 0.
    """
    q = np.asarray(q, np.float64)
    out = np.zeros((T * P, np.shape(v)[1]))
    for f in range(T):
        out[f * P:(f + 1) * P] = attend_rows(q[f * P:(f + 1) * P], k, v, P, frames_of(f), scale)
    return out


def attend_rows(q_rows, k, v, P, frames, scale=None):
    """Softmax attention of the given query rows over every key of `frames`
    (frame g = tokens g*P .. g*P+P-1 of k, v); zeros when `frames` is empty."""
    q_rows = np.asarray(q_rows, np.float64)
    d = q_rows.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    if not frames:
        return np.zeros((q_rows.shape[0], np.shape(v)[1]))
    idx = np.concatenate([np.arange(g * P, (g + 1) * P) for g in frames])
    kk = np.asarray(k[idx], np.float64)
    vv = np.asarray(v[idx], np.float64)
    z = scale * (q_rows @ kk.T)
    z -= z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ vv) / e.sum(axis=1, keepdims=True)


def frame_softmax_lse2(q, k, T, P, frames_of, scale=None):
    """Per query row, the log2 of its softmax denominator,
    log2 sum_j exp(scale q_i . k_j), over the keys of its frame set (the
    log-sum-exp that tiled exact attention carries per row, long-context page,
    section 03, here in log2 units); 0 for a row with no key frame.

    q, k: [T*P, d] float64 of one (batch, head); frames_of as in
    frame_softmax_attention. Returns [T*P]."""
    q = np.asarray(q, np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.zeros(T * P)
    for f in range(T):
        frames = frames_of(f)
        if not frames:
            continue
        idx = np.concatenate([np.arange(g * P, (g + 1) * P) for g in frames])
        z = scale * (q[f * P:(f + 1) * P] @ np.asarray(k[idx], np.float64).T)
        zm = z.max(axis=1)
        out[f * P:(f + 1) * P] = (zm + np.log(np.exp(z - zm[:, None]).sum(axis=1))) / np.log(2.0)
    return out


def swa(q, k, v, T, P, W, scale=None):
    return frame_softmax_attention(q, k, v, T, P, lambda f: swa_frames(f, W), scale)


def dswa(q, k, v, T, P, dil, taps, scale=None):
    return frame_softmax_attention(q, k, v, T, P, lambda f: dswa_frames(f, dil, taps), scale)


# ---------------------------------------------------------------------------
# gated delta rule memory
# ---------------------------------------------------------------------------

def l2norm_rows(x, eps=L2_EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)


def gdn_recurrent(q, k, v, a, b, S0=None, l2norm=True):
    """Gated delta rule, one token at a time (the reference of record).

    S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t.

    Decay first, then correct: the state is scaled by the gate a_t (the decay
    gate alpha_t of the recurrence quoted on the Kairos related-work page,
    row A), and the association stored under k_t is erased before v_t is
    written (long-context page, section 06: the delta rule and its gated
    form). S is [d_v, d_k]; q, k: [L, d_k]; v: [L, d_v]; a, b: [L].
    Returns (o [L, d_v], S_L).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if l2norm:
        q, k = l2norm_rows(q), l2norm_rows(k)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.empty((L, dv))
    for t in range(L):
        kt = k[t]
        erase = np.outer(S @ kt, kt)                 # what S currently stores under k_t
        S = a[t] * (S - b[t] * erase) + b[t] * np.outer(v[t], kt)
        o[t] = S @ q[t]
    return o, S


def gdn_chunked(q, k, v, a, b, C, S0=None, l2norm=True):
    """Gated delta rule in chunked (UT / WY) form; equals gdn_recurrent.

    Derivation (our own, from the recurrence above; the long-context page,
    sections 02 and 06, says chunkwise-parallel and recurrent forms of such a
    state are equivalent algorithms). Inside one chunk of n tokens with start
    state S0, write S_i = a_i S_{i-1} + u_i k_i^T with
    u_i = b_i (v_i - a_i S_{i-1} k_i), and let g_i = sum_{j<=i} log a_j,
    gamma_i = exp(g_i). Unrolling gives
        (I + A) U = diag(b) V - diag(b gamma) K S0^T,
        A_ij = b_i exp(g_i - g_j) (k_i . k_j)   for j < i,
    so with T = (I + A)^-1, W = T diag(b gamma) K and U' = T diag(b) V:
        U   = U' - W S0^T
        O   = diag(gamma) Q S0^T + (exp(g_i - g_j) q_i . k_j)_{j<=i} U
        S_n = gamma_n S0 + U^T diag(gamma_n / gamma) K.
    Chunks start at token 0 of the call; the last one may be shorter.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if l2norm:
        q, k = l2norm_rows(q), l2norm_rows(k)
    L, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    o = np.empty((L, dv))
    with np.errstate(divide="ignore"):
        loga = np.maximum(np.log(a), LOG_A_FLOOR)
    for s in range(0, L, C):
        e = min(s + C, L)
        n = e - s
        K, Q, V, bc = k[s:e], q[s:e], v[s:e], b[s:e]
        g = np.cumsum(loga[s:e])
        gam = np.exp(g)
        lower = np.tril(np.ones((n, n), bool))
        ratio = np.where(lower, np.exp(np.where(lower, g[:, None] - g[None, :], 0.0)), 0.0)
        A = np.tril(bc[:, None] * ratio * (K @ K.T), -1)
        IA = np.eye(n) + A
        Wm = solve_triangular(IA, (bc * gam)[:, None] * K, lower=True, unit_diagonal=True)
        Up = solve_triangular(IA, bc[:, None] * V, lower=True, unit_diagonal=True)
        U = Up - Wm @ S.T
        Aqk = ratio * (Q @ K.T)
        o[s:e] = gam[:, None] * (Q @ S.T) + Aqk @ U
        S = gam[-1] * S + U.T @ (np.exp(g[-1] - g)[:, None] * K)
    return o, S


def gates_from_logits(xa, xb):
    """Decay and write gates from raw logits (optional reading; the pages name
    the gates but not how a layer produces them): a = sigmoid(x_a),
    b = sigmoid(x_b), in the form that does not overflow for either sign."""
    def sig(x):
        x = np.asarray(x, np.float64)
        e = np.exp(-np.abs(x))
        return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return sig(xa), sig(xb)


# ---------------------------------------------------------------------------
# rotary position embedding of the softmax branches (optional)
# ---------------------------------------------------------------------------
#
# The pages say the local branches are sliding windows over latent frames and
# name no positional scheme. Reading taken for the optional rotary embedding:
# positions are three-dimensional, (absolute latent frame, row, column) with
# token p of a frame at row p // grid_w, column p % grid_w; the d/2 coordinate
# pairs (x[2i], x[2i+1]) are complex numbers rotated by angle pos * theta^(-j/n)
# where the first d/8 pairs follow the frame, the next half of the rest the
# row, the others the column, j is the pair's index within its axis and n the
# number of pairs of that axis. It applies to q and k of SWA and DSWA only; the
# memory branch reads q and k without positions.

def rope_axis_pairs(d):
    """Pairs of a head of size d given to the (frame, row, column) axes."""
    n = d // 2
    nt = d // 8
    nh = (n - nt) // 2
    return nt, nh, n - nt - nh


def rope_positions(T, P, grid_w, f0=0):
    """(frame, row, column) of the T*P tokens of frames f0 .. f0+T-1, [T*P, 3]."""
    t = np.arange(T * P)
    p = t % P
    return np.stack([f0 + t // P, p // grid_w, p % grid_w], axis=1).astype(np.float64)


def rope(x, pos, theta):
    """Rotate each token's coordinate pairs by its position (reading above).
    x [n_tokens, d], pos [n_tokens, 3]."""
    x = np.asarray(x, np.float64)
    d = x.shape[1]
    nt, nh, nw = rope_axis_pairs(d)
    out = np.empty_like(x)
    for i in range(d // 2):
        if i < nt:
            axis, j, n = 0, i, nt
        elif i < nt + nh:
            axis, j, n = 1, i - nt, nh
        else:
            axis, j, n = 2, i - nt - nh, nw
        ang = pos[:, axis] * float(theta) ** (-j / n)
        z = (x[:, 2 * i] + 1j * x[:, 2 * i + 1]) * np.exp(1j * ang)
        out[:, 2 * i] = z.real
        out[:, 2 * i + 1] = z.imag
    return out


# ---------------------------------------------------------------------------
# whole operator
# ---------------------------------------------------------------------------

def hlta_head(q, k, v, a, b, w3, T, P, W, dil, taps, C, scale=None, S0=None, gdn="chunked", rope_cfg=None,
              gate_logits=False):
    """HLTA forward of one (batch, head): returns o_swa, o_dswa, o_gdn, o_mix, S_out.
    rope_cfg = (theta, grid_w): rotary embedding of the softmax branches' q, k.
    gate_logits: a and b are logits (the memory uses their logistic function)."""
    if gate_logits:
        a, b = gates_from_logits(a, b)
    qa, ka = q, k
    if rope_cfg is not None:
        theta, grid_w = rope_cfg
        pos = rope_positions(T, P, grid_w)
        qa, ka = rope(q, pos, theta), rope(k, pos, theta)
    o_swa = swa(qa, ka, v, T, P, W, scale)
    o_dswa = dswa(qa, ka, v, T, P, dil, taps, scale)
    if gdn == "chunked":
        o_gdn, S = gdn_chunked(q, k, v, a, b, C, S0)
    else:
        o_gdn, S = gdn_recurrent(q, k, v, a, b, S0)
    w3 = np.asarray(w3, np.float64)
    o_mix = w3[0] * o_swa + w3[1] * o_dswa + w3[2] * o_gdn
    return o_swa, o_dswa, o_gdn, o_mix, S


def hlta_forward(q, k, v, a, b, w, T, P, W, dil, taps, C, scale=None, S0=None, gdn="chunked",
                 heads=None, rope_cfg=None, gate_logits=False):
    """HLTA forward over [B, L, H, d] inputs; returns float64 arrays in the same
    layout (o_* [B, L, H, d], S_out [B, H, d_v, d_k]). heads: optional list of
    (b, h) to compute (others stay zero)."""
    B, L, H, d = np.shape(q)
    dv = np.shape(v)[3]
    outs = [np.zeros((B, L, H, dv)) for _ in range(4)]
    S_out = np.zeros((B, H, dv, d))
    todo = heads if heads is not None else [(bi, hi) for bi in range(B) for hi in range(H)]
    for bi, hi in todo:
        s0 = None if S0 is None else S0[bi, hi]
        res = hlta_head(q[bi, :, hi], k[bi, :, hi], v[bi, :, hi], a[bi, :, hi], b[bi, :, hi],
                        w[hi], T, P, W, dil, taps, C, scale, s0, gdn, rope_cfg, gate_logits)
        for o, r in zip(outs, res[:4]):
            o[bi, :, hi] = r
        S_out[bi, hi] = res[4]
    return (*outs, S_out)


# ---------------------------------------------------------------------------
# streaming: one latent frame at a time
# ---------------------------------------------------------------------------

class StreamHead:
    """Streaming HLTA of one (rollout, head): keeps the state S and the K/V of
    past frames, and appends one latent frame per step without recomputing the
    clip (Kairos article on zhichai.net, section 2.3: streaming tokens for
    incremental generation; long-context page, section 02: a recurrent twin of
    the parallel form for decoding)."""

    def __init__(self, P, W, dil, taps, C, scale=None, S0=None, rope_cfg=None, gate_logits=False):
        self.P, self.W, self.dil, self.taps, self.C = P, W, dil, taps, C
        self.scale = scale
        self.rope_cfg = rope_cfg   # (theta, grid_w): past keys are kept rotated
        self.gate_logits = gate_logits
        self.S0 = None if S0 is None else np.array(S0, np.float64)
        self.k = {}
        self.v = {}
        self.f = 0

    def _rot(self, x, f):
        if self.rope_cfg is None:
            return np.asarray(x, np.float64)
        theta, grid_w = self.rope_cfg
        return rope(x, rope_positions(1, self.P, grid_w, f0=f), theta)

    def load_prefix(self, k, v, frames, S):
        for j in range(frames):
            self.k[j] = self._rot(k[j * self.P:(j + 1) * self.P], j)
            self.v[j] = np.asarray(v[j * self.P:(j + 1) * self.P], np.float64)
        self.f = frames
        self.S0 = np.array(S, np.float64)

    def step(self, q, k, v, a, b, w3, commit=True):
        P, f = self.P, self.f
        q = np.asarray(q, np.float64)
        kf = np.asarray(k, np.float64)
        vf = np.asarray(v, np.float64)
        scale = 1.0 / np.sqrt(q.shape[1]) if self.scale is None else self.scale

        qr, kr = self._rot(q, f), self._rot(kf, f)

        def attend(frames):
            if not frames:
                return np.zeros((P, vf.shape[1]))
            ks = np.concatenate([kr if g == f else self.k[g] for g in frames])
            vs = np.concatenate([vf if g == f else self.v[g] for g in frames])
            z = scale * (qr @ ks.T)
            z -= z.max(axis=1, keepdims=True)
            e = np.exp(z)
            return (e @ vs) / e.sum(axis=1, keepdims=True)

        o_swa = attend(swa_frames(f, self.W))
        o_dswa = attend(dswa_frames(f, self.dil, self.taps))
        if self.gate_logits:
            a, b = gates_from_logits(a, b)
        o_gdn, S = gdn_chunked(q, kf, vf, a, b, self.C, self.S0)
        w3 = np.asarray(w3, np.float64)
        o_mix = w3[0] * o_swa + w3[1] * o_dswa + w3[2] * o_gdn
        if commit:
            self.k[f], self.v[f] = kr, vf
            self.S0 = S
            self.f = f + 1
        return o_swa, o_dswa, o_gdn, o_mix


# ---------------------------------------------------------------------------
# backward: gradients of the operator (the training workload)
# ---------------------------------------------------------------------------
#
# Given the gradient of the mixed output, d_mix [B, L, H, d], the gradients of
# q, k, v, the gates, the mix weights and the start state. Every formula is the
# chain rule through the forward definitions above (no approximation); the
# pins compare them with central differences of those forward functions.

def attention_backward(q, k, v, do, T, P, frames_of, scale=None):
    """Gradients (dq, dk, dv) of the frame-block softmax attention
    o = frame_softmax_attention(q, k, v, T, P, frames_of) given do = dL/do.
    Per query frame f with keys K (its frame set): Z = s q K^T, Pm = softmax(Z),
    o = Pm V; dV += Pm^T do, dPm = do V^T, dZ = Pm * (dPm - rowsum(dPm * Pm)),
    dq = s dZ K, dK += s dZ^T q."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for f in range(T):
        frames = frames_of(f)
        if not frames:
            continue
        rows = slice(f * P, (f + 1) * P)
        idx = np.concatenate([np.arange(g * P, (g + 1) * P) for g in frames])
        z = scale * (q[rows] @ k[idx].T)
        z -= z.max(axis=1, keepdims=True)
        pm = np.exp(z)
        pm /= pm.sum(axis=1, keepdims=True)
        dv[idx] += pm.T @ do[rows]
        dpm = do[rows] @ v[idx].T
        dz = pm * (dpm - np.sum(dpm * pm, axis=1, keepdims=True))
        dq[rows] += scale * (dz @ k[idx])
        dk[idx] += scale * (dz.T @ q[rows])
    return dq, dk, dv


def gdn_recurrent_backward(q, k, v, a, b, do, S0=None, l2norm=True):
    """Gradients (dq, dk, dv, da, db, dS0) of the gated delta rule (gdn_recurrent)
    given do = dL/do_t, by running the recurrence backwards. With k^ = k/n(k),
    n(x) = sqrt(|x|^2 + eps), u = S_{t-1} k^, X = S_{t-1} - b u k^^T and
    S_t = a X + b v k^^T, o_t = S_t q^; for G = dL/dS_t (do_t q^^T plus what
    flows back from later tokens):
      dq^ = S_t^T do_t, da = <G, X>, dX = a G, dv = b G k^,
      db = v^T G k^ - u^T dX k^,  dk^ = b G^T v - b (S_{t-1}^T dX + dX^T S_{t-1}) k^,
      dL/dS_{t-1} = dX - b (dX k^) k^^T,
    and through the normalisation dx = dx^/n - x (x.dx^)/n^3."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    do = np.asarray(do, np.float64)
    L, dk_ = k.shape
    dvd = v.shape[1]
    qh, kh = (l2norm_rows(q), l2norm_rows(k)) if l2norm else (q, k)
    S = np.zeros((dvd, dk_)) if S0 is None else np.array(S0, np.float64)
    states = [S]
    for t in range(L):
        u = S @ kh[t]
        S = a[t] * (S - b[t] * np.outer(u, kh[t])) + b[t] * np.outer(v[t], kh[t])
        states.append(S)
    dqh, dkh = np.zeros_like(qh), np.zeros_like(kh)
    dv, da, db = np.zeros_like(v), np.zeros(L), np.zeros(L)
    G = np.zeros((dvd, dk_))
    for t in range(L - 1, -1, -1):
        St, Sp = states[t + 1], states[t]
        G = G + np.outer(do[t], qh[t])
        dqh[t] = St.T @ do[t]
        u = Sp @ kh[t]
        X = Sp - b[t] * np.outer(u, kh[t])
        da[t] = np.sum(G * X)
        dX = a[t] * G
        dv[t] = b[t] * (G @ kh[t])
        db[t] = v[t] @ G @ kh[t] - u @ dX @ kh[t]
        dkh[t] = b[t] * (G.T @ v[t]) - b[t] * (Sp.T @ dX + dX.T @ Sp) @ kh[t]
        G = dX - b[t] * np.outer(dX @ kh[t], kh[t])
    def through_norm(x, dxh):
        n = np.sqrt(np.sum(x * x, axis=1, keepdims=True) + L2_EPS)
        return dxh / n - x * np.sum(x * dxh, axis=1, keepdims=True) / n ** 3
    dq = through_norm(q, dqh) if l2norm else dqh
    dk = through_norm(k, dkh) if l2norm else dkh
    return dq, dk, dv, da, db, G


def hlta_backward(q, k, v, a, b, w, d_mix, T, P, W, dil, taps, scale=None, S0=None):
    """Gradients of L = <d_mix, o_mix> for inputs [B, L, H, d]: returns dq, dk,
    dv [B, L, H, d], da, db [B, L, H], dw [H, 3], dS0 [B, H, d_v, d_k]. The
    branch gradients are do_i = w[h, i] * d_mix; dw[h, i] = <d_mix, o_i>."""
    q = np.asarray(q, np.float64)
    B, Lt, H, d = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros(np.shape(v))
    da, db = np.zeros((B, Lt, H)), np.zeros((B, Lt, H))
    dw, dS0 = np.zeros((H, 3)), np.zeros((B, H, np.shape(v)[3], d))
    for bi in range(B):
        for hi in range(H):
            qh, kh, vh = q[bi, :, hi], np.asarray(k[bi, :, hi], np.float64), np.asarray(v[bi, :, hi], np.float64)
            g = np.asarray(d_mix[bi, :, hi], np.float64)
            w3 = np.asarray(w[hi], np.float64)
            s0 = None if S0 is None else S0[bi, hi]
            o_swa = swa(qh, kh, vh, T, P, W, scale)
            o_dswa = dswa(qh, kh, vh, T, P, dil, taps, scale)
            o_gdn, _ = gdn_recurrent(qh, kh, vh, a[bi, :, hi], b[bi, :, hi], s0)
            dw[hi] += [np.sum(g * o_swa), np.sum(g * o_dswa), np.sum(g * o_gdn)]
            for wi, fo in ((w3[0], lambda f: swa_frames(f, W)), (w3[1], lambda f: dswa_frames(f, dil, taps))):
                gq, gk, gv = attention_backward(qh, kh, vh, wi * g, T, P, fo, scale)
                dq[bi, :, hi] += gq
                dk[bi, :, hi] += gk
                dv[bi, :, hi] += gv
            gq, gk, gv, ga, gb, gS = gdn_recurrent_backward(qh, kh, vh, a[bi, :, hi], b[bi, :, hi], w3[2] * g, s0)
            dq[bi, :, hi] += gq
            dk[bi, :, hi] += gk
            dv[bi, :, hi] += gv
            da[bi, :, hi] = ga
            db[bi, :, hi] = gb
            dS0[bi, hi] = gS
    return dq, dk, dv, da, db, dw, dS0


# ---------------------------------------------------------------------------
# FP8 (e4m3) variant of the softmax branches: input quantisation
# ---------------------------------------------------------------------------
#
# The pages mention low-precision attention without a method. The variant
# implemented: q, k, v quantised per (batch row, head) to the e4m3 format
# (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
# value 448; subnormals down to 2^-9) with the scale s = max|x| / 448, codes
# = e4m3(x / s) rounded to nearest, ties to even, after clamping to +-448;
# x / s and s itself are taken in float32 (both sides decide the codes in the
# same precision). The attention then runs on the decoded values times s.

E4M3_MAX = 448.0


def e4m3_encode(x):
    """Nearest e4m3 code (ties to even) of float values already within +-448."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0)
    code = np.zeros(x.shape, np.int64)
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)          # 0 .. 8 (8 = smallest normal)
    nrm = ~sub
    e = np.floor(np.log2(a[nrm])).astype(np.int64)
    m = np.rint((a[nrm] / 2.0 ** e - 1.0) * 8.0).astype(np.int64)       # 0 .. 8
    e = np.where(m == 8, e + 1, e)
    m = np.where(m == 8, 0, m)
    code[nrm] = (e + 7) * 8 + m
    return (code | sign).astype(np.uint8)


def e4m3_decode(code):
    """Value of e4m3 codes (0x7f / 0xff, the NaN codes, are never produced here)."""
    c = np.asarray(code, np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    return np.where(c & 0x80, -mag, mag)


def quantize_e4m3(x):
    """Per-(batch row, head) e4m3 quantisation of x [B, L, H, d]: returns codes
    (uint8, same shape) and the float32 scales [B, H]."""
    x32 = np.asarray(x, np.float32)
    amax = np.abs(x32).max(axis=(1, 3))                                # [B, H]
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x32 / scale[:, None, :, None]).astype(np.float32)
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3_encode(y), scale


def dequantize_e4m3(code, scale):
    """Decoded values times their (batch row, head) scale, float64."""
    return e4m3_decode(code) * np.asarray(scale, np.float64)[:, None, :, None]


# ---------------------------------------------------------------------------
# comparison
# ---------------------------------------------------------------------------

def rel_l2(x, ref):
    """||x - ref||_2 / ||ref||_2 in float64 (0 when both are zero)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm((x - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
