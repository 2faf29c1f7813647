"""Pins for the float64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a closed form, an invariant, a library
routine computing the same sub-step, a brute-force evaluation at 50 digits,
a hand-worked example, or an equality the pages state (token-by-token ==
single-shot == split prefill; rollback-then-replay == never drafted).  The
mutant tests at the end plant plausible mistakes in a copy of the recurrence
and show that the pins catch them.
"""
import json
import math
import os

from dataclasses import replace

import mpmath
import numpy as np
import pytest

from oracle import kda_oracle as O
from hybrid_linear_attention_kda_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def rand_unit(shape, rng=RNG):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_recurrence_inputs(T, H, dk, dv, rng, lb=-5.0):
    q = rand_unit((T, H, dk), rng)
    k = rand_unit((T, H, dk), rng)
    v = rng.standard_normal((T, H, dv))
    g = lb / (1 + np.exp(-rng.standard_normal((T, H, dk)) * 2))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def params_for(wl, inp):
    return O.KdaParams(H=wl.H, dk=wl.dk, dv=wl.dv, conv_w=inp["conv_w"], A_log=inp["A_log"],
                       dt_bias=inp["dt_bias"], norm_w=inp["norm_w"], lb=inp["lb"], scale=inp["scale"],
                       gate=inp["gate"])


# ---------------------------------------------------------------------------
# Sub-steps against library routines and closed forms
# ---------------------------------------------------------------------------

def test_conv_equals_numpy_convolve():
    T, C, W = 11, 7, 4
    x = RNG.standard_normal((T, C))
    cs = RNG.standard_normal((C, W - 1))
    cw = RNG.standard_normal((C, W))
    y, new_cs = O.causal_depthwise_conv(x, cs, cw)
    xt = np.concatenate([cs.T, x], axis=0)
    for c in range(C):
        ref = np.convolve(xt[:, c], cw[c, ::-1], mode="valid")
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_array_equal(new_cs, x[T - (W - 1):].T)


def test_conv_causal_and_state_carry():
    # Output at t depends only on inputs <= t; two calls carrying the conv state equal one call.
    T, C, W = 9, 5, 4
    x = RNG.standard_normal((T, C))
    cs = np.zeros((C, W - 1))
    cw = RNG.standard_normal((C, W))
    y, _ = O.causal_depthwise_conv(x, cs, cw)
    x2 = x.copy()
    x2[6:] += 100.0
    y2, _ = O.causal_depthwise_conv(x2, cs, cw)
    np.testing.assert_array_equal(y[:6], y2[:6])
    ya, csa = O.causal_depthwise_conv(x[:4], cs, cw)
    yb, csb = O.causal_depthwise_conv(x[4:], csa, cw)
    np.testing.assert_array_equal(np.concatenate([ya, yb]), y)


def test_silu_and_sigmoid_against_closed_forms():
    x = np.linspace(-30, 30, 101)
    # The tanh spelling cancels for large negative x, so it is compared in absolute terms, and
    # mpmath pins the small tail in relative terms.
    np.testing.assert_allclose(O.sigmoid(x), 0.5 * (1 + np.tanh(x / 2)), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(O.silu(x), x * 0.5 * (1 + np.tanh(x / 2)), rtol=1e-13, atol=1e-15)
    mpmath.mp.dps = 40
    for xv in (-30.0, -12.5, -3.0, 0.0, 2.0, 25.0):
        ref = 1 / (1 + mpmath.exp(-mpmath.mpf(xv)))
        assert abs(O.sigmoid(np.array([xv]))[0] - float(ref)) <= 1e-15 * float(ref)
    assert O.sigmoid(np.array([-1000.0]))[0] == 0.0 and O.sigmoid(np.array([1000.0]))[0] == 1.0


def test_l2_normalize_eps_is_max_form():
    x = RNG.standard_normal((4, 16))
    np.testing.assert_allclose(O.l2_normalize(x, 1e-6), x / np.linalg.norm(x, axis=-1, keepdims=True),
                               rtol=1e-15)
    tiny = np.full((1, 16), 1e-9)  # ||tiny|| = 4e-9 < eps: divided by eps itself
    np.testing.assert_allclose(O.l2_normalize(tiny, 1e-6), tiny / 1e-6, rtol=1e-15)
    assert np.all(O.l2_normalize(np.zeros((2, 8)), 1e-6) == 0.0)
    # The other spelling sqrt(sum + eps) differs from max(||x||, eps) by about eps/(2 sum).
    y = RNG.standard_normal(128)
    alt = y / np.sqrt(np.sum(y * y) + 1e-6)
    rel = np.max(np.abs(O.l2_normalize(y, 1e-6) - alt)) / np.max(np.abs(alt))
    assert 0 < rel < 1e-6 / np.sum(y * y)


def test_decay_gate_range_bias_order_and_head_broadcast():
    H, dk, T = 3, 4, 5
    f = RNG.standard_normal((T, H * dk))
    A_log = RNG.uniform(0, math.log(16), H)
    dt = RNG.normal(0, 0.1, H * dk)
    g = O.decay_gate(f, A_log, dt, -5.0, H, dk)
    assert g.shape == (T, H, dk)
    assert np.all(g < 0) and np.all(g > -5.0)
    # dt_bias is per channel, added before the reshape: channel h*dk+i feeds head h, key channel i.
    dt2 = dt.copy()
    dt2[1 * dk + 2] += 3.0
    g2 = O.decay_gate(f, A_log, dt2, -5.0, H, dk)
    changed = np.argwhere(np.any(g2 != g, axis=0))
    assert changed.tolist() == [[1, 2]]
    # A is per head: raising A_log[h] changes only head h.
    A2 = A_log.copy()
    A2[2] += 0.5
    g3 = O.decay_gate(f, A2, dt, -5.0, H, dk)
    assert np.all(g3[:, :2] == g[:, :2]) and np.any(g3[:, 2] != g[:, 2])
    # Closed form at f + dt_bias = 0: g = lb/2 for every A.
    g0 = O.decay_gate(np.zeros((1, H * dk)), A_log, np.zeros(H * dk), -5.0, H, dk)
    np.testing.assert_array_equal(g0, np.full((1, H, dk), -2.5))
    # lb = 0 switches the decay off exactly (alpha = 1).
    assert np.all(np.exp(O.decay_gate(f, A_log, dt, 0.0, H, dk)) == 1.0)


def _gate_hand_worked_passes(gate_fn):
    # tests/golden/gate_hand_worked.json: A = exp(A_log) an integer, A (f + dt_bias) an integer
    d = json.load(open(os.path.join(GOLDEN, "gate_hand_worked.json")))
    for c in d["cases"]:
        g = gate_fn(np.array([[c["f"]]]), np.array([c["A_log"]]), np.array([c["dt_bias"]]), c["lb"], 1, 1)
        if not abs(float(g[0, 0, 0]) - c["g"]) <= 1e-14 * abs(c["g"]):
            return False
    return True


def _gate_monotone_passes(gate_fn):
    # With lb < 0 and a positive rate A: a larger f + dt_bias decays more (g falls towards lb), a
    # smaller one decays less (g rises towards 0); for f + dt_bias > 0 a larger A_log decays more.
    z = np.linspace(-3.0, 3.0, 25)[:, None]
    g = gate_fn(z, np.array([0.7]), np.zeros(1), -5.0, 1, 1)[:, 0, 0]
    if not np.all(np.diff(g) < 0):
        return False
    A_logs = np.linspace(-1.0, 2.5, 8)
    gA = np.array([gate_fn(np.array([[0.4]]), np.array([a]), np.zeros(1), -5.0, 1, 1)[0, 0, 0] for a in A_logs])
    return bool(np.all(np.diff(gA) < 0))


def _gate_through_layer_passes():
    # beta = 0 leaves only the decay: one token from S0 = 1 gives S1 = exp(g) with g the hand-worked
    # case 0 value (A_log = ln 2, f + dt_bias = 0.5, lb = -5) on every channel
    d = json.load(open(os.path.join(GOLDEN, "gate_hand_worked.json")))["cases"][0]
    H, dk, dv, W = 1, 4, 4, 1
    c = 2 * H * dk + H * dv
    p = O.KdaParams(H=H, dk=dk, dv=dv, conv_w=np.ones((c, W)), A_log=np.array([d["A_log"]]),
                    dt_bias=np.full(H * dk, d["dt_bias"]), norm_w=np.ones(dv), lb=d["lb"], scale=1.0)
    r = O.kda_layer(p, RNG.standard_normal((1, 1, c)), np.full((1, 1, H * dk), d["f"]), np.zeros((1, 1, H)),
                    np.zeros((1, 1, H * dv)), np.ones((1, H, dk, dv)), np.zeros((1, c, 0)))
    return bool(np.allclose(r["state"], math.exp(d["g"]), rtol=1e-14, atol=0))


def test_decay_gate_hand_worked_values():
    assert _gate_hand_worked_passes(O.decay_gate)


def test_decay_gate_is_monotone_in_the_pre_activation_and_the_rate():
    assert _gate_monotone_passes(O.decay_gate)


def test_decay_gate_hand_worked_value_through_the_layer():
    assert _gate_through_layer_passes()


def test_softplus_against_mpmath_and_tails():
    mpmath.mp.dps = 40
    for xv in (-700.0, -40.0, -5.0, -1.0, 0.0, 1e-8, 0.5, 3.0, 30.0, 700.0):
        ref = mpmath.log1p(mpmath.exp(mpmath.mpf(xv)))
        assert abs(O.softplus(np.array([xv]))[0] - float(ref)) <= 1e-15 * float(ref)
    # softplus(x) - softplus(-x) = x (the function is x plus its mirror image)
    x = RNG.standard_normal(50) * 20
    np.testing.assert_allclose(O.softplus(x) - O.softplus(-x), x, rtol=1e-13, atol=1e-13)


def test_softplus_gate_closed_forms_bias_order_and_head_broadcast():
    # The branch taken without a lower bound (llama.cpp PR #27754, metadata commit); reading:
    # g = -exp(A_log[h]) * softplus(f + dt_bias).
    H, dk, T = 3, 4, 5
    A_log = RNG.uniform(0, math.log(16), H)
    A = np.exp(A_log)
    # f + dt_bias = 0: g = -A ln 2 (A outside the softplus: -softplus(A z) would give -ln 2)
    g0 = O.decay_gate(np.zeros((1, H * dk)), A_log, np.zeros(H * dk), float("nan"), H, dk, "softplus")
    np.testing.assert_allclose(g0[0], np.repeat(-A * math.log(2.0), dk).reshape(H, dk), rtol=1e-15)
    # large arguments: g = -A (z + e^-z) to rounding; unbounded below (no clamp at any lb)
    z = 30.0
    gz = O.decay_gate(np.full((1, H * dk), z), A_log, np.zeros(H * dk), float("nan"), H, dk, "softplus")
    np.testing.assert_allclose(gz[0], np.repeat(-A * (z + math.exp(-z)), dk).reshape(H, dk), rtol=1e-15)
    g500 = O.decay_gate(np.full((1, H * dk), 500.0), A_log, np.zeros(H * dk), float("nan"), H, dk, "softplus")
    assert np.all(g500 <= -500.0)
    # very negative arguments: g = -A e^z (nearly no decay, still strictly negative)
    gn = O.decay_gate(np.full((1, H * dk), -40.0), A_log, np.zeros(H * dk), float("nan"), H, dk, "softplus")
    np.testing.assert_allclose(gn[0], np.repeat(-A * math.exp(-40.0), dk).reshape(H, dk), rtol=1e-12)
    assert np.all(gn < 0)
    # dt_bias per channel before the reshape; A per head
    f = RNG.standard_normal((T, H * dk))
    dt = RNG.normal(0, 0.1, H * dk)
    g = O.decay_gate(f, A_log, dt, float("nan"), H, dk, "softplus")
    dt2 = dt.copy()
    dt2[2 * dk + 1] -= 2.0
    g2 = O.decay_gate(f, A_log, dt2, float("nan"), H, dk, "softplus")
    assert np.argwhere(np.any(g2 != g, axis=0)).tolist() == [[2, 1]]
    A2 = A_log.copy()
    A2[0] += 0.25
    g3 = O.decay_gate(f, A2, dt, float("nan"), H, dk, "softplus")
    assert np.all(g3[:, 1:] == g[:, 1:]) and np.all(g3[:, 0] < g[:, 0])


def test_softplus_branch_follows_the_bound_being_absent():
    wl, inp, p = _tiny(6, gate="softplus")
    assert math.isnan(p.lb) and p.gate == "softplus"
    O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])
    for bad in (replace(p, lb=-5.0), replace(p, gate="tanh"), replace(p, gate="sigmoid")):
        with pytest.raises(ValueError):
            O.kda_layer(bad, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])


def test_softplus_strong_decay_forgets_the_state():
    # f + dt_bias = 300: g = -300 A <= -300 per token, alpha ~ 1e-130: each token starts from an empty
    # state, so o_t = scale * beta_t (q^_t . k^_t) v_t with the normalised q^, k (the one-token closed form)
    wl, inp, p = _tiny(7, gate="softplus")
    f = np.full_like(inp["f"], 300.0)
    S0 = RNG.standard_normal(inp["state0"].shape)
    r = O.kda_layer(p, inp["qkv"], f, inp["beta"], inp["g_out"], S0, inp["conv_state0"])
    q, k, v, g, _ = O.prologue(p, inp["qkv"][0], f[0], inp["conv_state0"][0])
    assert np.all(g <= -300.0)
    beta = inp["beta"][0]
    o_ref = np.einsum("thc,thc->th", q, k)[:, :, None] * beta[:, :, None] * v
    np.testing.assert_allclose(r["o"][0], o_ref, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("chunk", [16, 64])
def test_softplus_chunked_equals_token_and_split_is_exact(chunk):
    # the chunked spelling with pairwise decay factors stays finite under unbounded decay
    wl, inp, p = _tiny(45, gate="softplus")
    S0 = RNG.standard_normal(inp["state0"].shape)
    tok = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, inp["conv_state0"])
    ch = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, inp["conv_state0"],
                     form="chunked", chunk=chunk)
    assert np.all(np.isfinite(ch["out"]))
    np.testing.assert_allclose(ch["out"], tok["out"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ch["state"], tok["state"], rtol=1e-10, atol=1e-12)
    a, b = I.split_tokens(inp, 0, 20), I.split_tokens(inp, 20, 45)
    r1 = O.kda_layer(p, a["qkv"], a["f"], a["beta"], a["g_out"], S0, inp["conv_state0"])
    r2 = O.kda_layer(p, b["qkv"], b["f"], b["beta"], b["g_out"], r1["state"], r1["conv_state"])
    np.testing.assert_array_equal(np.concatenate([r1["out"], r2["out"]], axis=1), tok["out"])


def test_gated_rmsnorm_closed_forms():
    o = RNG.standard_normal((3, 2, 16))
    y = O.gated_rmsnorm(o, np.full(o.shape, 800.0), np.ones(16), 0.0)  # sigmoid(800) == 1
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-14)
    c = 0.01
    y = O.gated_rmsnorm(np.full((1, 1, 8), c), np.zeros((1, 1, 8)), np.full(8, 2.0), 1e-5)
    np.testing.assert_allclose(y, np.full((1, 1, 8), c / math.sqrt(c * c + 1e-5) * 2.0 * 0.5), rtol=1e-14)


def test_ut_solve_equals_numpy_solve():
    L, n = 16, 5
    A = np.tril(RNG.standard_normal((L, L)) * 0.3, -1)
    rhs = RNG.standard_normal((L, n))
    np.testing.assert_allclose(O.ut_forward_substitution(A, rhs),
                               np.linalg.solve(np.eye(L) + A, rhs), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# The recurrence: closed forms, invariants, brute force
# ---------------------------------------------------------------------------

def test_hand_worked_example():
    d = json.load(open(os.path.join(GOLDEN, "hand_worked_recurrence.json")))
    q, k, v = (np.array(d[x])[:, None, :] for x in ("q", "k", "v"))
    g = np.log(np.array(d["alpha"]))[:, None, :]
    beta = np.array(d["beta"])[:, None]
    o, S, states = O.recurrence_token(q, k, v, g, beta, np.zeros((1, 2, 2)), record_states=True)
    np.testing.assert_allclose(o[:, 0], np.array(d["o"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(states[:, 0], np.array(d["states"]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 0.3])
def test_one_token_from_zero_state(scale):
    # o = beta (q.k) v for one token from S = 0 (with q scaled by `scale`).
    H, dk, dv = 3, 8, 6
    q, k, v, g, beta = rand_recurrence_inputs(1, H, dk, dv, RNG)
    o, S, _ = O.recurrence_token(scale * q, k, v, g, beta, np.zeros((H, dk, dv)))
    qk = np.sum(q[0] * k[0], axis=-1)
    np.testing.assert_allclose(o[0], scale * beta[0][:, None] * qk[:, None] * v[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, beta[0][:, None, None] * k[0][:, :, None] * v[0][:, None, :], rtol=1e-15)


def _one_token_layer_passes(scale):
    # Identity conv (only the current-token tap = 1): q = scale silu(x_q)/||.||, k = silu(x_k)/||.||,
    # v = silu(x_v); one token from a zero state gives o = beta (q.k) v = scale beta cos(q^, k^) v, so
    # the scale shows in o only when it is applied after the normalisation
    H, dk, dv, W = 2, 8, 8, 4
    c = 2 * H * dk + H * dv
    conv_w = np.zeros((c, W))
    conv_w[:, W - 1] = 1.0
    p = O.KdaParams(H=H, dk=dk, dv=dv, conv_w=conv_w, A_log=np.zeros(H), dt_bias=np.zeros(H * dk),
                    norm_w=np.ones(dv), lb=-5.0, scale=scale)
    rng = np.random.default_rng(41)
    x = rng.standard_normal((1, 1, c))
    beta = np.array([[[0.3, 0.8]]])
    r = O.kda_layer(p, x, rng.standard_normal((1, 1, H * dk)), beta, np.zeros((1, 1, H * dv)),
                    np.zeros((1, H, dk, dv)), np.zeros((1, c, W - 1)))
    s = x[0, 0] / (1 + np.exp(-x[0, 0]))
    for h in range(H):
        qh = s[h * dk:(h + 1) * dk]
        kh = s[H * dk + h * dk: H * dk + (h + 1) * dk]
        vh = s[2 * H * dk + h * dv: 2 * H * dk + (h + 1) * dv]
        expect = scale * beta[0, 0, h] * (qh @ kh) / (np.linalg.norm(qh) * np.linalg.norm(kh)) * vh
        if not np.allclose(r["o"][0, 0, h], expect, rtol=1e-13, atol=1e-15):
            return False
    return True


def _query_norm_passes():
    # after the prologue every query has length `scale` and every key length 1 (conv outputs far
    # above the 1e-6 clamp)
    wl, inp, p = _tiny(9)
    p = replace(p, scale=0.3)
    q, k, _, _, _ = O.prologue(p, inp["qkv"][0], inp["f"][0], inp["conv_state0"][0])
    return bool(np.allclose(np.linalg.norm(q, axis=-1), 0.3, rtol=1e-14, atol=0)
                and np.allclose(np.linalg.norm(k, axis=-1), 1.0, rtol=1e-14, atol=0))


@pytest.mark.parametrize("scale", [1.0, 0.3])
def test_one_token_from_zero_state_through_the_layer(scale):
    assert _one_token_layer_passes(scale)


def test_prologue_query_length_is_the_scale():
    assert _query_norm_passes()


def test_beta_zero_decay_zero_leaves_state_bit_exact():
    H, dk, dv, T = 2, 8, 8, 7
    q, k, v, g, beta = rand_recurrence_inputs(T, H, dk, dv, RNG)
    S0 = RNG.standard_normal((H, dk, dv))
    _, S, _ = O.recurrence_token(q, k, v, np.zeros_like(g), np.zeros_like(beta), S0)
    np.testing.assert_array_equal(S, S0)


def test_beta_zero_decay_zero_through_the_layer():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=9)
    inp = I.generate(wl)
    p = params_for(wl, inp)
    p.lb = 0.0
    S0 = RNG.standard_normal((1, wl.H, wl.dk, wl.dv))
    r = O.kda_layer(p, inp["qkv"], inp["f"], np.zeros_like(inp["beta"]), inp["g_out"], S0, inp["conv_state0"])
    np.testing.assert_array_equal(r["state"], S0)


def test_beta_zero_is_pure_key_axis_decay():
    H, dk, dv, T = 2, 8, 5, 6
    q, k, v, g, beta = rand_recurrence_inputs(T, H, dk, dv, RNG)
    S0 = RNG.standard_normal((H, dk, dv))
    _, S, _ = O.recurrence_token(q, k, v, g, np.zeros_like(beta), S0)
    np.testing.assert_allclose(S, np.prod(np.exp(g), axis=0)[:, :, None] * S0, rtol=1e-13)


def test_delta_rule_recall_with_beta_one():
    # beta = 1 and ||k|| = 1: right after the update the state maps k_t to v_t exactly.
    H, dk, dv, T = 2, 8, 8, 6
    q, k, v, g, beta = rand_recurrence_inputs(T, H, dk, dv, RNG)
    _, _, states = O.recurrence_token(q, k, v, g, np.ones_like(beta), RNG.standard_normal((H, dk, dv)),
                                      record_states=True)
    for t in range(T):
        np.testing.assert_allclose(np.einsum("hk,hkv->hv", k[t], states[t]), v[t], rtol=1e-12, atol=1e-12)


def test_one_hot_keys_reduce_to_gated_linear_attention():
    # Distinct one-hot keys: the delta term vanishes and
    #   o_t = sum_{j<=t} beta_j q_t[c_j] prod_{j<s<=t} alpha_s[c_j] v_j   (per-channel decay on the key axis)
    H, dk, dv, T = 1, 8, 5, 6
    chans = [3, 0, 6, 1, 7, 2]
    k = np.zeros((T, H, dk))
    for t, c in enumerate(chans):
        k[t, 0, c] = 1.0
    q = RNG.standard_normal((T, H, dk))
    v = RNG.standard_normal((T, H, dv))
    g = -RNG.uniform(0.1, 2.0, (T, H, dk))
    beta = RNG.uniform(0.1, 0.9, (T, H))
    o, _, _ = O.recurrence_token(q, k, v, g, beta, np.zeros((H, dk, dv)))
    alpha = np.exp(g)
    for t in range(T):
        ref = np.zeros(dv)
        for j in range(t + 1):
            c = chans[j]
            ref += beta[j, 0] * q[t, 0, c] * np.prod(alpha[j + 1:t + 1, 0, c]) * v[j, 0]
        np.testing.assert_allclose(o[t, 0], ref, rtol=1e-13, atol=1e-14)


def test_linear_in_initial_state_and_values():
    H, dk, dv, T = 2, 6, 4, 5
    q, k, v, g, beta = rand_recurrence_inputs(T, H, dk, dv, RNG)
    S1, S2 = RNG.standard_normal((2, H, dk, dv))
    v2 = RNG.standard_normal(v.shape)
    a, b = 0.7, -1.3
    o1, F1, _ = O.recurrence_token(q, k, v, g, beta, S1)
    o2, F2, _ = O.recurrence_token(q, k, v2, g, beta, S2)
    o3, F3, _ = O.recurrence_token(q, k, a * v + b * v2, g, beta, a * S1 + b * S2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(F3, a * F1 + b * F2, rtol=1e-12, atol=1e-12)


def _brute_force_mp(q, k, v, alpha, beta, S0, digits=50):
    """Affine transition form at 50 digits: S_t = (I - b k k^T) Diag(alpha) S_{t-1} + b k v^T."""
    mpmath.mp.dps = digits
    T, dk = k.shape
    dv = v.shape[1]
    S = mpmath.matrix(S0.tolist())
    outs = []
    for t in range(T):
        kk = mpmath.matrix(k[t].tolist())
        P = mpmath.eye(dk) - mpmath.mpf(beta[t]) * (kk * kk.T)
        D = mpmath.diag([mpmath.mpf(a) for a in alpha[t]])
        S = P * D * S + mpmath.mpf(beta[t]) * kk * mpmath.matrix([v[t].tolist()])
        outs.append([float(x) for x in (S.T * mpmath.matrix(q[t].tolist()))])
    return np.array(outs), np.array([[float(S[i, j]) for j in range(dv)] for i in range(dk)])


@pytest.mark.parametrize("T,dk,dv", [(8, 4, 4), (7, 4, 3), (5, 3, 4)])
def test_brute_force_at_50_digits(T, dk, dv):
    rng = np.random.default_rng(T * 100 + dk * 10 + dv)
    q, k, v, g, beta = rand_recurrence_inputs(T, 1, dk, dv, rng)
    S0 = rng.standard_normal((1, dk, dv))
    o, S, _ = O.recurrence_token(q, k, v, g, beta, S0)
    o_mp, S_mp = _brute_force_mp(q[:, 0], k[:, 0], v[:, 0], np.exp(g[:, 0]), beta[:, 0], S0[0])
    np.testing.assert_allclose(o[:, 0], o_mp, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S[0], S_mp, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# Equalities the pages state
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_chunked_form_equals_token_form(chunk):
    H, dk, dv, T = 2, 16, 12, 45  # ragged last chunk for every chunk size
    rng = np.random.default_rng(chunk)
    q, k, v, g, beta = rand_recurrence_inputs(T, H, dk, dv, rng)
    S0 = rng.standard_normal((H, dk, dv))
    o_t, S_t, _ = O.recurrence_token(q, k, v, g, beta, S0)
    o_c, S_c = O.recurrence_chunked(q, k, v, g, beta, S0, chunk)
    scale_o = np.max(np.abs(o_t))
    assert np.max(np.abs(o_c - o_t)) / scale_o < 1e-12
    assert np.max(np.abs(S_c - S_t)) / np.max(np.abs(S_t)) < 1e-12


def test_chunked_form_strong_decay_does_not_overflow():
    # g at the bound everywhere: exp(Gam) underflows towards 1e-139 over 64 tokens; pairwise factors stay <= 1.
    H, dk, dv, T = 1, 8, 8, 128
    rng = np.random.default_rng(7)
    q, k, v, _, beta = rand_recurrence_inputs(T, H, dk, dv, rng)
    g = np.full((T, H, dk), -4.999)
    S0 = rng.standard_normal((H, dk, dv))
    o_t, S_t, _ = O.recurrence_token(q, k, v, g, beta, S0)
    o_c, S_c = O.recurrence_chunked(q, k, v, g, beta, S0, 64)
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_t, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(S_c, S_t, rtol=1e-10, atol=1e-13)


def _tiny(T=12, **kw):
    wl = I.WORKLOADS["tiny_fp32"].with_(T=T, **kw)
    inp = I.generate(wl)
    return wl, inp, params_for(wl, inp)


def test_split_prefill_5_plus_7_is_bit_exact():
    # glm53-flash-mlx README, tests: chunked prefill 5+7 vs single-shot max|delta| 0.
    wl, inp, p = _tiny(12)
    full = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])
    a = I.split_tokens(inp, 0, 5)
    b = I.split_tokens(inp, 5, 12)
    r1 = O.kda_layer(p, a["qkv"], a["f"], a["beta"], a["g_out"], inp["state0"], inp["conv_state0"])
    r2 = O.kda_layer(p, b["qkv"], b["f"], b["beta"], b["g_out"], r1["state"], r1["conv_state"])
    np.testing.assert_array_equal(np.concatenate([r1["out"], r2["out"]], axis=1), full["out"])
    np.testing.assert_array_equal(r2["state"], full["state"])
    np.testing.assert_array_equal(r2["conv_state"], full["conv_state"])


def test_token_by_token_decode_equals_single_forward():
    # glm53-flash-mlx README, tests: incremental decode equals a single forward.
    wl, inp, p = _tiny(10)
    full = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])
    S, cs, outs = inp["state0"], inp["conv_state0"], []
    for t in range(10):
        s = I.split_tokens(inp, t, t + 1)
        r = O.kda_layer(p, s["qkv"], s["f"], s["beta"], s["g_out"], S, cs)
        S, cs = r["state"], r["conv_state"]
        outs.append(r["out"])
    np.testing.assert_array_equal(np.concatenate(outs, axis=1), full["out"])
    np.testing.assert_array_equal(S, full["state"])


def test_layer_chunked_equals_layer_token():
    wl, inp, p = _tiny(64)
    a = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])
    b = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"],
                    form="chunked", chunk=16)
    assert np.max(np.abs(a["out"] - b["out"])) < 1e-12
    assert np.max(np.abs(a["state"] - b["state"])) < 1e-12


def test_verify_snapshots_equal_m_token_prefills():
    wl, inp, p = _tiny(8, B=2)
    S0 = RNG.standard_normal((2, wl.H, wl.dk, wl.dv))
    cs0 = RNG.standard_normal(inp["conv_state0"].shape)
    v = O.kda_verify(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    for m in range(1, 9):
        s = I.split_tokens(inp, 0, m)
        r = O.kda_layer(p, s["qkv"], s["f"], s["beta"], s["g_out"], S0, cs0)
        np.testing.assert_array_equal(v["snaps"][:, m - 1], r["state"])
        np.testing.assert_array_equal(v["out"][:, :m], r["out"])


@pytest.mark.parametrize("m", list(range(9)))
def test_rollback_then_replay_equals_never_drafted(m):
    # Draft 8 tokens, keep m, roll back, then decode one more (true) token.  The result must equal
    # running the m accepted tokens plus that token with no draft at all.
    wl, inp, p = _tiny(9, B=1)
    S0 = RNG.standard_normal((1, wl.H, wl.dk, wl.dv))
    cs0 = RNG.standard_normal(inp["conv_state0"].shape)
    draft = I.split_tokens(inp, 0, 8)
    v = O.kda_verify(p, draft["qkv"], draft["f"], draft["beta"], draft["g_out"], S0, cs0)
    S, cs = O.kda_rollback(p, [m], v["snaps"], draft["qkv"], S0, cs0)
    nxt = I.split_tokens(inp, 8, 9)
    after = O.kda_layer(p, nxt["qkv"], nxt["f"], nxt["beta"], nxt["g_out"], S, cs)
    idx = list(range(m)) + [8]
    ref = O.kda_layer(p, inp["qkv"][:, idx], inp["f"][:, idx], inp["beta"][:, idx], inp["g_out"][:, idx], S0, cs0)
    np.testing.assert_array_equal(after["out"][:, 0], ref["out"][:, -1])
    np.testing.assert_array_equal(after["state"], ref["state"])
    np.testing.assert_array_equal(after["conv_state"], ref["conv_state"])


def test_rollback_rejects_out_of_range():
    wl, inp, p = _tiny(8)
    snaps = np.zeros((1, 8, wl.H, wl.dk, wl.dv))
    with pytest.raises(ValueError):
        O.kda_rollback(p, [9], snaps, inp["qkv"], inp["state0"], inp["conv_state0"])


def test_verify_tape_outputs_equal_snapshot_verify():
    wl, inp, p = _tiny(8, B=2)
    S0 = RNG.standard_normal((2, wl.H, wl.dk, wl.dv))
    cs0 = RNG.standard_normal(inp["conv_state0"].shape)
    v = O.kda_verify(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    vt = O.kda_verify_tape(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    np.testing.assert_array_equal(vt["out"], v["out"])
    # the tape's key is the normalised key and its decay exp(g), straight from the prologue
    q, k, vv, g, _ = O.prologue(p, inp["qkv"][0], inp["f"][0], cs0[0])
    np.testing.assert_array_equal(vt["tape"][0, :, :, 1], k)
    np.testing.assert_array_equal(vt["tape"][0, :, :, 0], np.exp(g))


@pytest.mark.parametrize("m", list(range(9)))
def test_tape_commit_equals_snapshot_rollback(m):
    # The replayed state is the verify pass's own state after m tokens (same operations in the
    # same order), and the conv window is the rollback's.
    wl, inp, p = _tiny(8, B=2)
    S0 = RNG.standard_normal((2, wl.H, wl.dk, wl.dv))
    cs0 = RNG.standard_normal(inp["conv_state0"].shape)
    v = O.kda_verify(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    vt = O.kda_verify_tape(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    acc = [m, 8 - m]
    S1, c1 = O.kda_rollback(p, acc, v["snaps"], inp["qkv"], S0, cs0)
    S2, c2 = O.kda_commit_tape(p, acc, vt["tape"], inp["qkv"], S0, cs0)
    np.testing.assert_array_equal(S2, S1)
    np.testing.assert_array_equal(c2, c1)


def test_tape_closed_forms():
    # beta = 0: every u is zero and the commit is the pure key-axis decay prod_t alpha_t of S0;
    # one token from a zero state: u = beta v.
    wl, inp, p = _tiny(6, B=1)
    S0 = RNG.standard_normal((1, wl.H, wl.dk, wl.dv))
    cs0 = inp["conv_state0"]
    z = np.zeros_like(inp["beta"])
    vt = O.kda_verify_tape(p, inp["qkv"], inp["f"], z, inp["g_out"], S0, cs0)
    assert np.all(vt["tape"][:, :, :, 2] == 0.0)
    S, _ = O.kda_commit_tape(p, [6], vt["tape"], inp["qkv"], S0, cs0)
    decay = np.prod(vt["tape"][0, :, :, 0], axis=0)  # [H, dk]
    np.testing.assert_allclose(S[0], decay[:, :, None] * S0[0], rtol=1e-13, atol=0)
    vt1 = O.kda_verify_tape(p, inp["qkv"][:, :1], inp["f"][:, :1], inp["beta"][:, :1], inp["g_out"][:, :1],
                            np.zeros_like(S0), cs0)
    _, _, vv, _, _ = O.prologue(p, inp["qkv"][0, :1], inp["f"][0, :1], cs0[0])
    np.testing.assert_allclose(vt1["tape"][0, 0, :, 2], inp["beta"][0, 0][:, None] * vv[0], rtol=1e-15, atol=0)


def test_commit_tape_rejects_out_of_range():
    wl, inp, p = _tiny(8)
    tape = np.zeros((1, 8, wl.H, 3, wl.dk))
    with pytest.raises(ValueError):
        O.kda_commit_tape(p, [9], tape, inp["qkv"], inp["state0"], inp["conv_state0"])


def _packed(inp, B, T):
    return {k: inp[k].reshape(B * T, -1) for k in ("qkv", "f", "beta", "g_out")}


def test_varlen_equal_lengths_equals_batched_layer():
    wl, inp, p = _tiny(12, B=3)
    S0 = RNG.standard_normal((3, wl.H, wl.dk, wl.dv))
    cs0 = RNG.standard_normal(inp["conv_state0"].shape)
    full = O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], S0, cs0)
    pk = _packed(inp, 3, 12)
    v = O.kda_prefill_varlen(p, [0, 12, 24, 36], None, pk["qkv"], pk["f"], pk["beta"], pk["g_out"], S0, cs0)
    np.testing.assert_array_equal(v["out"], full["out"].reshape(36, -1))
    np.testing.assert_array_equal(v["state"], full["state"])
    np.testing.assert_array_equal(v["conv_state"], full["conv_state"])


def test_varlen_sequences_are_independent_of_order_and_slots():
    # each sequence is one call on its own slot: permuting the packing and the slot assignment
    # moves results around and changes nothing else; empty sequences and unnamed slots are untouched
    wl, inp, p = _tiny(30, B=1)
    pool = RNG.standard_normal((5, wl.H, wl.dk, wl.dv))
    cpool = RNG.standard_normal((5, wl.c_qkv, wl.W - 1))
    pk = _packed(inp, 1, 30)
    lens = [7, 0, 16, 7]
    cu = I.cu_seqlens(lens)
    v1 = O.kda_prefill_varlen(p, cu, [3, 1, 0, 4], pk["qkv"], pk["f"], pk["beta"], pk["g_out"], pool, cpool)
    np.testing.assert_array_equal(v1["state"][[1, 2]], pool[[1, 2]])
    np.testing.assert_array_equal(v1["conv_state"][[1, 2]], cpool[[1, 2]])
    # sequence 2 (tokens 7..22, slot 0) alone, as a plain layer call
    r = O.kda_layer(p, inp["qkv"][:, 7:23], inp["f"][:, 7:23], inp["beta"][:, 7:23], inp["g_out"][:, 7:23],
                    pool[None, 0], cpool[None, 0])
    np.testing.assert_array_equal(v1["out"][7:23], r["out"][0])
    np.testing.assert_array_equal(v1["state"][0], r["state"][0])
    # reversed packing order with the same slots per sequence
    order = [3, 2, 1, 0]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
    cu2 = I.cu_seqlens([lens[i] for i in order])
    v2 = O.kda_prefill_varlen(p, cu2, [[3, 1, 0, 4][i] for i in order], pk["qkv"][idx], pk["f"][idx],
                              pk["beta"][idx], pk["g_out"][idx], pool, cpool)
    np.testing.assert_array_equal(v2["out"], v1["out"][idx])
    np.testing.assert_array_equal(v2["state"], v1["state"])
    np.testing.assert_array_equal(v2["conv_state"], v1["conv_state"])


@pytest.mark.parametrize("cu,slots", [([1, 3], None), ([0, 4, 2], None), ([0, 2, 4], [0, 0]), ([0, 2, 4], [0, 9])])
def test_varlen_rejects_bad_tables(cu, slots):
    wl, inp, p = _tiny(4, B=1)
    pk = _packed(inp, 1, 4)
    pool = np.zeros((3, wl.H, wl.dk, wl.dv))
    with pytest.raises(ValueError):
        O.kda_prefill_varlen(p, cu, slots, pk["qkv"], pk["f"], pk["beta"], pk["g_out"], pool,
                             np.zeros((3, wl.c_qkv, wl.W - 1)))


def _proj_weights(H, d, r, hidden, rng):
    n = 3 * H * d + 2 * r + H
    return (rng.standard_normal((n, hidden)), rng.standard_normal((H * d, r)), rng.standard_normal((H * d, r)))


def test_projection_one_hot_rows_select_weight_columns():
    # x = identity: row i of every output is what weight column i maps to; the low-rank path equals
    # the product of its two Linear maps taken the other way round (associativity)
    H, d, r, hidden = 2, 16, 8, 12
    rng = np.random.default_rng(5)
    w_in, w_fb, w_gb = _proj_weights(H, d, r, hidden, rng)
    out = O.kda_input_projection(np.eye(hidden), w_in, w_fb, w_gb, H, d, r)
    HD = H * d
    np.testing.assert_array_equal(out["qkv"], w_in[:3 * HD].T)
    np.testing.assert_allclose(out["f"], (w_fb @ w_in[3 * HD:3 * HD + r]).T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["g_out"], (w_gb @ w_in[3 * HD + r:3 * HD + 2 * r]).T, rtol=1e-12, atol=1e-12)
    b = w_in[3 * HD + 2 * r:].T
    np.testing.assert_allclose(out["beta"], 0.5 + 0.5 * np.tanh(b / 2), rtol=1e-14)


def test_projection_zero_and_linearity():
    H, d, r, hidden = 2, 16, 8, 12
    rng = np.random.default_rng(6)
    w_in, w_fb, w_gb = _proj_weights(H, d, r, hidden, rng)
    z = O.kda_input_projection(np.zeros((3, hidden)), w_in, w_fb, w_gb, H, d, r)
    for k in ("qkv", "f", "g_out"):
        assert np.all(z[k] == 0.0)
    assert np.all(z["beta"] == 0.5)
    x = rng.standard_normal((5, hidden))
    a = O.kda_input_projection(x, w_in, w_fb, w_gb, H, d, r)
    b = O.kda_input_projection(2.0 * x, w_in, w_fb, w_gb, H, d, r)
    for k in ("qkv", "f", "g_out"):
        np.testing.assert_allclose(b[k], 2.0 * a[k], rtol=1e-13, atol=1e-13)


def test_missing_gate_lower_bound_is_an_error():
    wl, inp, p = _tiny(4)
    p.lb = float("nan")
    with pytest.raises(ValueError):
        O.kda_layer(p, inp["qkv"], inp["f"], inp["beta"], inp["g_out"], inp["state0"], inp["conv_state0"])


# ---------------------------------------------------------------------------
# Mutants: plausible mistakes planted in a copy of the recurrence must fail a pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def rec(q, k, v, g, beta, S0):
        S = np.array(S0, dtype=np.float64).copy()
        T = k.shape[0]
        o = np.zeros((T,) + v.shape[1:])
        for t in range(T):
            a = np.exp(g[t])
            if kind == "value_axis":
                S = S * a[:, None, :]          # decays the value axis (needs dk == dv)
            else:
                S = a[:, :, None] * S
            kS = np.einsum("hk,hkv->hv", k[t], S)
            sign = 1.0 if kind == "plus_sign" else -1.0
            u = beta[t][:, None] * (v[t] + sign * kS)
            if kind == "output_before_update":
                o[t] = np.einsum("hk,hkv->hv", q[t], S)
            S = S + k[t][:, :, None] * u[:, None, :]
            if kind != "output_before_update":
                o[t] = np.einsum("hk,hkv->hv", q[t], S)
        return o, S
    return rec


def _hand_worked_passes(rec):
    d = json.load(open(os.path.join(GOLDEN, "hand_worked_recurrence.json")))
    q, k, v = (np.array(d[x])[:, None, :] for x in ("q", "k", "v"))
    g = np.log(np.array(d["alpha"]))[:, None, :]
    o, _ = rec(q, k, v, g, np.array(d["beta"])[:, None], np.zeros((1, 2, 2)))
    return np.allclose(o[:, 0], np.array(d["o"]), atol=1e-12)


def _brute_force_passes(rec):
    rng = np.random.default_rng(99)
    q, k, v, g, beta = rand_recurrence_inputs(6, 1, 4, 4, rng)
    S0 = rng.standard_normal((1, 4, 4))
    o, S = rec(q, k, v, g, beta, S0)
    o_mp, S_mp = _brute_force_mp(q[:, 0], k[:, 0], v[:, 0], np.exp(g[:, 0]), beta[:, 0], S0[0], digits=30)
    return np.allclose(o[:, 0], o_mp, atol=1e-10) and np.allclose(S[0], S_mp, atol=1e-10)


def test_unmutated_copy_passes_the_pins():
    assert _hand_worked_passes(_mutant("none"))
    assert _brute_force_passes(_mutant("none"))


@pytest.mark.parametrize("kind", ["value_axis", "plus_sign", "output_before_update"])
def test_pins_catch_planted_mistakes(kind):
    rec = _mutant(kind)
    assert not _hand_worked_passes(rec)
    assert not _brute_force_passes(rec)


def _mutant_gate(kind):
    # copies of the bounded gate with a planted mistake in the rate A
    def gate(f, A_log, dt_bias, lb, H, dk, kind_=None):
        f = np.asarray(f, dtype=np.float64)
        z = (f + np.asarray(dt_bias, dtype=np.float64)[None, :]).reshape(f.shape[0], H, dk)
        A_log = np.asarray(A_log, dtype=np.float64)
        A = {"A_is_A_log": A_log, "A_negative": -np.exp(A_log)}[kind][None, :, None]
        return float(lb) / (1.0 + np.exp(-A * z))
    return gate


def _mutant_prologue_scale_before_norm():
    real = O.prologue

    def prologue(p, qkv, f, conv_state):
        q, k, v, g, cs = real(replace(p, scale=1.0), qkv, f, conv_state)
        # the mistake: scale the raw query, then normalise it (the scale cancels)
        return O.l2_normalize(p.scale * q, p.l2_eps), k, v, g, cs
    return prologue


@pytest.mark.parametrize("kind", ["A_is_A_log", "A_negative"])
def test_gate_pins_catch_planted_mistakes(kind, monkeypatch):
    mut = _mutant_gate(kind)
    assert not _gate_hand_worked_passes(mut)
    if kind == "A_negative":
        assert not _gate_monotone_passes(mut)
    monkeypatch.setattr(O, "decay_gate", mut)
    assert not _gate_through_layer_passes()


def test_scale_pins_catch_scale_before_the_norm(monkeypatch):
    assert _one_token_layer_passes(0.3) and _query_norm_passes()
    monkeypatch.setattr(O, "prologue", _mutant_prologue_scale_before_norm())
    assert not _one_token_layer_passes(0.3)
    assert not _query_norm_passes()


def test_scalar_gate_makes_key_and_value_axis_agree():
    # Gated DeltaNet special case (llama.cpp PR #27754, KDA commit): with one decay per head the
    # key-axis and value-axis spellings coincide; with per-channel decay they do not.
    rng = np.random.default_rng(3)
    q, k, v, g, beta = rand_recurrence_inputs(6, 2, 8, 8, rng)
    g_scalar = np.repeat(g[:, :, :1], 8, axis=2)
    S0 = rng.standard_normal((2, 8, 8))
    a, _ = _mutant("none")(q, k, v, g_scalar, beta, S0)
    b, _ = _mutant("value_axis")(q, k, v, g_scalar, beta, S0)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)
    a, _ = _mutant("none")(q, k, v, g, beta, S0)
    b, _ = _mutant("value_axis")(q, k, v, g, beta, S0)
    assert np.max(np.abs(a - b)) > 1e-3
