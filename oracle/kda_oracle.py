"""Float64 CPU oracle for the Kimi Delta Attention (KDA) layer.

TEST INFRASTRUCTURE ONLY.  This module is the checker the HIP library is
measured against.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import it; the library itself never does, and this
module imports nothing from the library (the two share no code).

Everything is computed in float64 from the exact values the GPU receives
(bf16 / fp32 inputs upcast exactly).  Nothing here is blocked, fused or
reordered beyond what the definition states, so each step can be checked
against the pages by eye.

Sources (the pages carry no equations for the layer; it is defined in prose):

* llama.cpp PR #27754 "model: add GLM-5-Next (GLM-5.3-Flash)", KDA commit
  message: one depthwise causal conv over the concatenated q|k|v channels
  with a single contiguous conv state; SiLU after the conv; q/k L2
  normalisation with a literal eps 1e-6 implemented as max(||x||, eps);
  a bounded-sigmoid per-channel decay gate with dt_bias added per channel
  before the reshape to heads and a per-head A broadcast, bounded below by
  kda.gate_lower_bound; f, g and beta taken from the pre-convolution hidden
  states; the state decays along the key axis, never the value axis; a gated
  output RMSNorm with a plain weight.
* Splash issue #740 "GLM-5.3-Flash family (glm5-next) with SSD expert
  streaming", maintainer answer: KDA is linear attention with a fixed-size
  recurrent state per head and no KV cache.
* dflash-mlx issue #63 "Add a Glm5NextTargetOps target adapter", "What the
  backend needs": the KDA recurrent state must support rollback of a
  speculative draft block (block size 8 for the DFlash2 drafter, Context).
* glm53-flash-mlx README, tests: token-by-token decode equals a single
  forward, and a chunked 5+7 prefill equals single-shot.
* glm53-flash-mlx README, port review: rms_norm_eps = 1e-5.

Readings taken where the pages leave a step open (each is also listed in the
design notes):

* gate:   g = lb * sigmoid(exp(A_log[h]) * (f + dt_bias)), alpha = exp(g),
          so the per-step log-decay lies in (lb, 0).
* softplus branch (llama.cpp PR #27754, metadata commit: kimi-k3 takes a
          softplus branch, a different function, when kda.gate_lower_bound is
          absent; the page gives no formula): g = -exp(A_log[h]) *
          softplus(f + dt_bias), the same parameters with the softplus in place
          of the bounded sigmoid and A as the decay rate; unbounded below.
* update: S <- Diag(alpha) S ; u = beta * (v - S^T k) ; S <- S + k u^T ;
          o = S^T q  (output read after the update).
* conv:   causal, no bias, tap W-1 multiplies the current token; the conv
          state holds the W-1 previous raw inputs, oldest first.
* q is multiplied by `scale` after its L2 normalisation.
* output: y = o / sqrt(mean(o^2) + rms_eps) * w * sigmoid(g_out), normalised
          over d_v per (token, head); w has shape [d_v], shared by heads.
* channel order of q|k|v: [q heads | k heads | v heads], each head's
          channels contiguous.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "KdaParams",
    "causal_depthwise_conv",
    "silu",
    "sigmoid",
    "softplus",
    "l2_normalize",
    "decay_gate",
    "gated_rmsnorm",
    "recurrence_token",
    "recurrence_chunked",
    "ut_forward_substitution",
    "prologue",
    "kda_layer",
    "kda_verify",
    "kda_rollback",
]


@dataclass
class KdaParams:
    """Per-layer parameters.  Arrays are converted to float64 on use.

    conv_w  [C_qkv, W]   depthwise conv taps, C_qkv = H*dk + H*dk + H*dv
    A_log   [H]          per-head log of the decay rate A
    dt_bias [H*dk]       per-channel bias added to f before the head reshape
    norm_w  [dv]         output RMSNorm weight (plain weight, not 1 + w)
    lb                   kda.gate_lower_bound (finite for the bounded gate; NaN,
                         i.e. absent, for the softplus branch)
    gate                 "sigmoid" (the bounded gate) or "softplus"
    """

    H: int
    dk: int
    dv: int
    conv_w: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    norm_w: np.ndarray
    lb: float
    scale: float = 1.0
    gate: str = "sigmoid"
    l2_eps: float = 1e-6
    rms_eps: float = 1e-5
    extra: dict = field(default_factory=dict)

    @property
    def c_qkv(self) -> int:
        return 2 * self.H * self.dk + self.H * self.dv

    @property
    def W(self) -> int:
        return int(np.asarray(self.conv_w).shape[1])


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------

def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-x) in float64 (saturates cleanly to 0 and 1)."""
    x = _f64(x)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def softplus(x: np.ndarray) -> np.ndarray:
    """ln(1 + e^x) in float64, written as max(x, 0) + ln(1 + e^-|x|) so that neither
    tail overflows (the two forms are equal for every x)."""
    x = _f64(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(y: np.ndarray) -> np.ndarray:
    """SiLU applied to the conv output (llama.cpp PR #27754, KDA commit)."""
    y = _f64(y)
    return y * sigmoid(y)


def causal_depthwise_conv(x: np.ndarray, conv_state: np.ndarray, conv_w: np.ndarray):
    """One depthwise causal conv over every q|k|v channel of one sequence.

    llama.cpp PR #27754, KDA commit: q|k|v are convolved as one depthwise
    kernel, so the conv state is a single contiguous block.

    x          [T, C]     raw pre-conv inputs of this call
    conv_state [C, W-1]   the W-1 raw inputs before x, oldest first
    conv_w     [C, W]     taps; tap W-1 multiplies the current token

    Returns y [T, C] with y[t, c] = sum_w conv_w[c, w] * xt[t + w, c] where
    xt = conv_state^T stacked above x, and the new conv state (the last W-1
    rows of xt, transposed back to [C, W-1]).
    """
    x = _f64(x)
    conv_state = _f64(conv_state)
    conv_w = _f64(conv_w)
    T = x.shape[0]
    W = conv_w.shape[1]
    xt = np.concatenate([conv_state.T, x], axis=0)  # [W-1+T, C]
    y = np.zeros_like(x)
    for w in range(W):
        y += conv_w[:, w][None, :] * xt[w:w + T]
    new_state = np.ascontiguousarray(xt[xt.shape[0] - (W - 1):].T)
    return y, new_state


def l2_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / max(||x||_2, eps) over the last axis.

    llama.cpp PR #27754, KDA commit: the q/k eps is a literal 1e-6 and the
    norm is clamped as max(sqrt(sum), eps).
    """
    x = _f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def decay_gate(f: np.ndarray, A_log: np.ndarray, dt_bias: np.ndarray, lb: float, H: int, dk: int,
               kind: str = "sigmoid"):
    """Per-channel log-decay g (the decay is alpha = exp(g)) for one sequence.

    llama.cpp PR #27754, KDA commit: a bounded-sigmoid decay gate; dt_bias is
    added per channel before the reshape to heads; A is per head and
    broadcast over the head's channels; kda.gate_lower_bound bounds it.

    f [T, H*dk] -> g [T, H, dk] with g = lb * sigmoid(exp(A_log[h]) * (f + dt_bias)),
    which lies in (lb, 0) for lb < 0.  kind "softplus" (the branch taken when
    the bound is absent, metadata commit): g = -exp(A_log[h]) * softplus(f + dt_bias),
    in (-inf, 0).
    """
    f = _f64(f)
    T = f.shape[0]
    z = (f + _f64(dt_bias)[None, :]).reshape(T, H, dk)
    A = np.exp(_f64(A_log))[None, :, None]
    if kind == "sigmoid":
        return float(lb) * sigmoid(A * z)
    if kind == "softplus":
        return -A * softplus(z)
    raise ValueError(f"unknown gate kind {kind!r}")


def gated_rmsnorm(o: np.ndarray, g_out: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Gated output RMSNorm with a plain weight (llama.cpp PR #27754, KDA commit).

    o [T, H, dv]; g_out [T, H, dv] gate logits; w [dv].
    y = o / sqrt(mean_dv(o^2) + eps) * w * sigmoid(g_out).
    """
    o = _f64(o)
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o * r * _f64(w)[None, None, :] * sigmoid(g_out)


# ---------------------------------------------------------------------------
# The recurrence
# ---------------------------------------------------------------------------

def recurrence_token(q, k, v, g, beta, S0, record_states: bool = False):
    """The KDA recurrence token by token, for every head at once.

    q, k [T, H, dk]; v [T, H, dv]; g [T, H, dk] log-decay; beta [T, H];
    S0 [H, dk, dv] (row = key channel).

    Per token t and head h:
        S <- Diag(exp(g_t)) S          decay along the key axis (rows)
        u  = beta_t (v_t - S^T k_t)     delta-rule correction
        S <- S + k_t u^T
        o_t = S^T q_t

    llama.cpp PR #27754, KDA commit: the decay is applied on the key axis,
    never on the value axis.  Returns (o [T,H,dv], S_T [H,dk,dv], states)
    where states [T,H,dk,dv] is the state after every token when
    record_states is set (else None).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    S = _f64(S0).copy()
    T, H, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    states = np.zeros((T, H, dk, dv)) if record_states else None
    for t in range(T):
        S = np.exp(g[t])[:, :, None] * S
        kS = np.einsum("hk,hkv->hv", k[t], S)
        u = beta[t][:, None] * (v[t] - kS)
        S = S + k[t][:, :, None] * u[:, None, :]
        o[t] = np.einsum("hk,hkv->hv", q[t], S)
        if record_states:
            states[t] = S
    return o, S, states


def recurrence_token_tape(q, k, v, g, beta, S0):
    """The token recurrence of recurrence_token, also returning each token's
    replay tape: alpha_t = exp(g_t) [H, dk] and u_t = beta_t (v_t - S'^T k_t)
    [H, dv], with S' the decayed state the update reads.

    With these the state after token t is Diag(alpha_t) S_{t-1} + k_t u_t^T, so
    an accepted prefix of a draft block can be re-applied to the live state
    without storing the state after every token (dflash-mlx issue #63, "What
    the backend needs": rollback of a speculative block).
    Returns (o [T,H,dv], S_T [H,dk,dv], alpha [T,H,dk], u [T,H,dv]).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    S = _f64(S0).copy()
    T, H, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    alpha = np.exp(g)
    us = np.zeros((T, H, dv))
    for t in range(T):
        S = alpha[t][:, :, None] * S
        kS = np.einsum("hk,hkv->hv", k[t], S)
        u = beta[t][:, None] * (v[t] - kS)
        S = S + k[t][:, :, None] * u[:, None, :]
        o[t] = np.einsum("hk,hkv->hv", q[t], S)
        us[t] = u
    return o, S, alpha, us


def ut_forward_substitution(A: np.ndarray, rhs: np.ndarray) -> np.ndarray:
    """Solve (I + A) X = rhs for strictly lower-triangular A by forward substitution.

    X[i] = rhs[i] - sum_{j<i} A[i, j] X[j].
    """
    A = _f64(A)
    X = _f64(rhs).copy()
    for i in range(X.shape[0]):
        X[i] = X[i] - A[i, :i] @ X[:i]
    return X


def recurrence_chunked(q, k, v, g, beta, S0, chunk: int):
    """The same recurrence in chunked WY/UT form (exact reformulation).

    The method's prefill is chunked with an intra-chunk WY/UT solve (the
    "chunked fallback" delta net of llama.cpp PR #27754, KDA commit, plays
    this role there).  Within a chunk of L tokens with inclusive cumulative
    log-decay Gam[i] = sum_{s<=i} g[s] (per key channel) and chunk-start
    state S:

        A_kk[i, j] = beta_i sum_c k_i[c] k_j[c] exp(Gam_i[c] - Gam_j[c])   (j < i)
        A_qk[i, j] =        sum_c q_i[c] k_j[c] exp(Gam_i[c] - Gam_j[c])   (j <= i)
        (I + A_kk) W  = beta * K * exp(Gam)
        (I + A_kk) Ut = beta * V
        U = Ut - W S
        O = (Q * exp(Gam)) S + A_qk U
        S <- Diag(exp(Gam_L)) S + (K * exp(Gam_L - Gam))^T U

    The pairwise factors exp(Gam_i - Gam_j) are formed directly (no
    factorisation), so nothing can overflow.  Returns (o [T,H,dv], S_T).
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    T, H, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    S_all = _f64(S0).copy()
    for h in range(H):
        S = S_all[h]
        for c0 in range(0, T, chunk):
            c1 = min(c0 + chunk, T)
            L = c1 - c0
            Q, K, V = q[c0:c1, h], k[c0:c1, h], v[c0:c1, h]
            b = beta[c0:c1, h]
            Gam = np.cumsum(g[c0:c1, h], axis=0)  # [L, dk]
            diff = Gam[:, None, :] - Gam[None, :, :]  # [i, j, c] = Gam_i - Gam_j
            i_idx = np.arange(L)[:, None]
            j_idx = np.arange(L)[None, :]
            strict = (j_idx < i_idx)[:, :, None]
            incl = (j_idx <= i_idx)[:, :, None]
            E_strict = np.exp(np.where(strict, diff, -np.inf))
            E_incl = np.exp(np.where(incl, diff, -np.inf))
            A_kk = b[:, None] * np.einsum("ic,jc,ijc->ij", K, K, E_strict)
            A_qk = np.einsum("ic,jc,ijc->ij", Q, K, E_incl)
            Wm = ut_forward_substitution(A_kk, b[:, None] * K * np.exp(Gam))
            Ut = ut_forward_substitution(A_kk, b[:, None] * V)
            U = Ut - Wm @ S
            o[c0:c1, h] = (Q * np.exp(Gam)) @ S + A_qk @ U
            S = np.exp(Gam[L - 1])[:, None] * S + (K * np.exp(Gam[L - 1][None, :] - Gam)).T @ U
        S_all[h] = S
    return o, S_all


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def prologue(p: KdaParams, qkv, f, conv_state):
    """Conv, SiLU, L2 normalisation, q scale and decay gate for one sequence.

    qkv [T, C_qkv] raw pre-conv inputs; f [T, H*dk]; conv_state [C_qkv, W-1].
    Returns (q, k, v, g, new_conv_state) with q, k [T,H,dk], v [T,H,dv],
    g [T,H,dk].  The gate is computed from f, which (like beta and g_out)
    comes from the pre-convolution hidden states, so the conv never touches it.
    """
    H, dk, dv = p.H, p.dk, p.dv
    T = np.asarray(qkv).shape[0]
    y, new_cs = causal_depthwise_conv(qkv, conv_state, p.conv_w)
    z = silu(y)
    q_hat = z[:, : H * dk].reshape(T, H, dk)
    k_hat = z[:, H * dk: 2 * H * dk].reshape(T, H, dk)
    v = z[:, 2 * H * dk:].reshape(T, H, dv)
    q = p.scale * l2_normalize(q_hat, p.l2_eps)
    k = l2_normalize(k_hat, p.l2_eps)
    g = decay_gate(f, p.A_log, p.dt_bias, p.lb, H, dk, p.gate)
    return q, k, v, g, new_cs


def _check_lb(p: KdaParams):
    """The branch follows the bound's presence (metadata commit): the bounded gate needs a
    finite kda.gate_lower_bound; the softplus branch is the one taken when it is absent (NaN)."""
    if p.gate == "sigmoid":
        if not np.isfinite(p.lb):
            raise ValueError("gate_lower_bound is required and must be finite")
    elif p.gate == "softplus":
        if not np.isnan(p.lb):
            raise ValueError("the softplus branch is the one without gate_lower_bound (pass NaN)")
    else:
        raise ValueError(f"unknown gate kind {p.gate!r}")


def kda_layer(p: KdaParams, qkv, f, beta, g_out, state, conv_state, *,
              form: str = "token", chunk: int = 64, record_states: bool = False):
    """One KDA layer call over a batch of sequences.

    qkv   [B, T, C_qkv]      raw q|k|v projections (pre-conv)
    f     [B, T, H*dk]       gate pre-activation
    beta  [B, T, H]          delta-rule step size, in (0, 1)
    g_out [B, T, H*dv]       output-gate logits
    state [B, H, dk, dv]     recurrent state (not modified)
    conv_state [B, C_qkv, W-1]

    Returns dict(out [B,T,H*dv], state, conv_state, o [B,T,H,dv] (pre-norm),
    states [B,T,H,dk,dv] when record_states).
    """
    _check_lb(p)
    qkv, f, beta, g_out = (_f64(a) for a in (qkv, f, beta, g_out))
    state, conv_state = _f64(state), _f64(conv_state)
    B, T, _ = qkv.shape
    H, dv = p.H, p.dv
    out = np.zeros((B, T, H * dv))
    o_all = np.zeros((B, T, H, dv))
    new_state = np.zeros_like(state)
    new_cs = np.zeros_like(conv_state)
    states = np.zeros((B, T, H, p.dk, dv)) if record_states else None
    for b in range(B):
        q, k, v, g, new_cs[b] = prologue(p, qkv[b], f[b], conv_state[b])
        if form == "token":
            o, S, st = recurrence_token(q, k, v, g, beta[b], state[b], record_states)
            if record_states:
                states[b] = st
        elif form == "chunked":
            if record_states:
                raise ValueError("per-token states come from the token form")
            o, S = recurrence_chunked(q, k, v, g, beta[b], state[b], chunk)
        else:
            raise ValueError(form)
        new_state[b] = S
        o_all[b] = o
        out[b] = gated_rmsnorm(o, g_out[b].reshape(T, H, dv), p.norm_w, p.rms_eps).reshape(T, H * dv)
    return {"out": out, "state": new_state, "conv_state": new_cs, "o": o_all, "states": states}


def kda_verify(p: KdaParams, qkv, f, beta, g_out, state, conv_state):
    """Verify a draft block: run T_d tokens from the live state and record the
    state after every token (the snapshots rollback restores).  The live state
    and conv state are left as they were.

    dflash-mlx issue #63, "What the backend needs": rollback of the KDA
    recurrent state; llama.cpp PR #27754, KDA commit: the conv state is one
    contiguous block so it can be snapshotted.

    Returns dict(out [B,T_d,H*dv], snaps [B,T_d,H,dk,dv]).
    """
    r = kda_layer(p, qkv, f, beta, g_out, state, conv_state, form="token", record_states=True)
    return {"out": r["out"], "snaps": r["states"]}


def kda_rollback(p: KdaParams, accepted, snaps, qkv_block, state, conv_state):
    """Commit the accepted prefix of a verified block.

    For each sequence b with m = accepted[b] in 0..T_d:
        state[b]      <- snaps[b, m-1]   (unchanged when m = 0)
        conv_state[b] <- the last W-1 rows of (conv_state[b] || qkv_block[b, :m])
    Returns (state, conv_state) as new float64 arrays.
    """
    snaps, qkv_block = _f64(snaps), _f64(qkv_block)
    state, conv_state = _f64(state).copy(), _f64(conv_state).copy()
    W = p.W
    T_d = snaps.shape[1]
    for b, m in enumerate(accepted):
        m = int(m)
        if m < 0 or m > T_d:
            raise ValueError("accepted prefix length out of range")
        if m == 0:
            continue
        state[b] = snaps[b, m - 1]
        xt = np.concatenate([conv_state[b].T, qkv_block[b, :m]], axis=0)
        conv_state[b] = xt[xt.shape[0] - (W - 1):].T
    return state, conv_state


def kda_verify_tape(p: KdaParams, qkv, f, beta, g_out, state, conv_state):
    """Verify a draft block recording a replay tape instead of snapshots.

    Same outputs as kda_verify.  tape[b, t, h] = (alpha_t, k_t, u_t): the
    token's decay exp(g_t), its normalised key and its delta-rule update, each
    of length d (d_k == d_v).  The live state and conv state are not modified.
    Returns dict(out [B,T_d,H*dv], tape [B,T_d,H,3,d]).
    """
    _check_lb(p)
    if p.dk != p.dv:
        raise ValueError("the replay tape needs d_k == d_v")
    qkv, f, beta, g_out = (_f64(a) for a in (qkv, f, beta, g_out))
    state, conv_state = _f64(state), _f64(conv_state)
    B, T, _ = qkv.shape
    H, d = p.H, p.dk
    out = np.zeros((B, T, H * d))
    tape = np.zeros((B, T, H, 3, d))
    for b in range(B):
        q, k, v, g, _cs = prologue(p, qkv[b], f[b], conv_state[b])
        o, _S, alpha, u = recurrence_token_tape(q, k, v, g, beta[b], state[b])
        tape[b, :, :, 0] = alpha
        tape[b, :, :, 1] = k
        tape[b, :, :, 2] = u
        out[b] = gated_rmsnorm(o, g_out[b].reshape(T, H, d), p.norm_w, p.rms_eps).reshape(T, H * d)
    return {"out": out, "tape": tape}


def kda_commit_tape(p: KdaParams, accepted, tape, qkv_block, state, conv_state):
    """Commit the accepted prefix of a block verified with a replay tape.

    For each sequence b with m = accepted[b] in 0..T_d:
        for t < m:  state[b] <- Diag(alpha_t) state[b] + k_t u_t^T
        conv_state[b] <- the last W-1 rows of (conv_state[b] || qkv_block[b, :m])
    state must be the state the verify call read.  Returns (state, conv_state)
    as new float64 arrays.
    """
    tape, qkv_block = _f64(tape), _f64(qkv_block)
    state, conv_state = _f64(state).copy(), _f64(conv_state).copy()
    W = p.W
    T_d = tape.shape[1]
    for b, m in enumerate(accepted):
        m = int(m)
        if m < 0 or m > T_d:
            raise ValueError("accepted prefix length out of range")
        if m == 0:
            continue
        S = state[b]
        for t in range(m):
            alpha, k, u = tape[b, t, :, 0], tape[b, t, :, 1], tape[b, t, :, 2]
            S = alpha[:, :, None] * S
            S = S + k[:, :, None] * u[:, None, :]
        state[b] = S
        xt = np.concatenate([conv_state[b].T, qkv_block[b, :m]], axis=0)
        conv_state[b] = xt[xt.shape[0] - (W - 1):].T
    return state, conv_state


def kda_prefill_varlen(p: KdaParams, cu_seqlens, slots, qkv, f, beta, g_out, state, conv_state, *,
                       form: str = "token", chunk: int = 64):
    """Sequences of different lengths packed along the token axis, each
    continuing the state held in its own slot of a state pool (the hybrid
    memory keeps one recurrent-state cell per sequence: llama.cpp PR #27754,
    KDA commit, n_rs_seq).  Sequence i is tokens cu_seqlens[i] ..
    cu_seqlens[i+1]-1 and is exactly one kda_layer call on its own.

    qkv [total, C_qkv], f [total, H*dk], beta [total, H], g_out [total, H*dv];
    state [num_slots, H, dk, dv], conv_state [num_slots, C_qkv, W-1];
    slots [N] distinct slot indices (None: slot i).  Slots not named, and the
    slots of empty sequences, are returned unchanged.
    Returns dict(out [total, H*dv], state, conv_state) as new float64 arrays.
    """
    cu = [int(c) for c in cu_seqlens]
    N = len(cu) - 1
    if N < 0 or cu[0] != 0 or any(cu[i + 1] < cu[i] for i in range(N)):
        raise ValueError("cu_seqlens must start at 0 and not decrease")
    state, conv_state = _f64(state).copy(), _f64(conv_state).copy()
    slots = list(range(N)) if slots is None else [int(s) for s in slots]
    if len(slots) != N or len(set(slots)) != N or any(s < 0 or s >= state.shape[0] for s in slots):
        raise ValueError("slots must be N distinct indices into the state pool")
    qkv, f, beta, g_out = (_f64(a) for a in (qkv, f, beta, g_out))
    out = np.zeros((cu[-1], p.H * p.dv))
    for i in range(N):
        a, e, s = cu[i], cu[i + 1], slots[i]
        if e == a:
            continue
        r = kda_layer(p, qkv[None, a:e], f[None, a:e], beta[None, a:e], g_out[None, a:e], state[None, s],
                      conv_state[None, s], form=form, chunk=chunk)
        out[a:e] = r["out"][0]
        state[s] = r["state"][0]
        conv_state[s] = r["conv_state"][0]
    return {"out": out, "state": state, "conv_state": conv_state}


def kda_input_projection(x, w_in, w_fb, w_gb, H: int, d: int, rank: int):
    """The step before the layer: the six input projections of the hidden states x [T, hidden].

    w_in [3*H*d + 2*rank + H, hidden] holds the q, k, v, f_a, g_a and b projections as one
    weight (rows in that order; the runtime fuses them into one matmul, glm53-flash-mlx README,
    quantization recipe).  f and the output gate are low rank, f = f_b(f_a x) and
    g_out = g_b(g_a x) (llama.cpp PR #27754, KDA commit); beta = sigmoid(b x).  Weights are
    Linear weights [out, in].  Returns dict(qkv [T, 3Hd], f [T, Hd], beta [T, H], g_out [T, Hd]).
    """
    x, w_in, w_fb, w_gb = (_f64(a) for a in (x, w_in, w_fb, w_gb))
    HD = H * d
    y = x @ w_in.T
    fa = y[:, 3 * HD:3 * HD + rank]
    ga = y[:, 3 * HD + rank:3 * HD + 2 * rank]
    return {"qkv": y[:, :3 * HD], "f": fa @ w_fb.T, "beta": sigmoid(y[:, 3 * HD + 2 * rank:]),
            "g_out": ga @ w_gb.T}
