"""Shared helpers for the GPU parity tests: run the oracle on a workload and
compare the library's results with it.

The metric is per tensor: max|x - ref| / max|ref| in float64.  Tolerances:
fp32 io 1e-5, bf16 io 2e-3 (outputs compared in fp32 output mode; bf16
output mode adds at most one bf16 rounding, 2^-9 of max|ref|).
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import kda_oracle as O
from hybrid_linear_attention_kda_amd import inputs as I

TOL = {"f32": 1e-5, "bf16": 2e-3}
TOL_BF16_OUT = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(x - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)


def params(wl: I.Workload, inp: dict) -> O.KdaParams:
    return O.KdaParams(H=wl.H, dk=wl.dk, dv=wl.dv, conv_w=inp["conv_w"], A_log=inp["A_log"],
                       dt_bias=inp["dt_bias"], norm_w=inp["norm_w"], lb=inp["lb"], scale=inp["scale"],
                       gate=inp["gate"], rms_eps=inp.get("rms_eps", 1e-5))


def oracle_layer(wl, inp, t0, t1, state, conv_state, form="token", record_states=False):
    tok = I.split_tokens(inp, t0, t1)
    return O.kda_layer(params(wl, inp), tok["qkv"], tok["f"], tok["beta"], tok["g_out"], state, conv_state,
                       form=form, chunk=wl.chunk, record_states=record_states)


_PREFILLED = {}


def oracle_prefilled(wl, inp, n_pre: int):
    """State and conv state after the workload's prefix tokens, computed by the
    oracle for the first n_pre sequences and assigned to sequence b from
    sequence b % n_pre (the step under test then continues that sequence
    with sequence b's own new tokens).  Kept per (workload, n_pre) for the
    other tests of the same session."""
    key = (wl, n_pre)
    if key not in _PREFILLED:
        sub_inp = dict(inp)
        for k in ("qkv", "f", "beta", "g_out"):
            sub_inp[k] = inp[k][:n_pre]
        r = oracle_layer(wl, sub_inp, 0, wl.prefix_T, inp["state0"][:n_pre], inp["conv_state0"][:n_pre])
        _PREFILLED[key] = (r["state"].astype(np.float32), r["conv_state"].astype(np.float32))
    st, cs = _PREFILLED[key]
    idx = np.arange(wl.B) % n_pre
    return st[idx], cs[idx]


def head_channels(wl, heads):
    """Indices of the given heads' channels in out [.., H*dv] and in qkv [.., 3*H*d]."""
    H, d = wl.H, wl.dk
    oc = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    qc = oc
    ch = np.concatenate([qc, qc + H * d, qc + 2 * H * d])
    return oc, ch
