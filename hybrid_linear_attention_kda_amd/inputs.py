"""Seeded synthetic inputs for the KDA layer workloads.

This module only draws random numbers and rounds them to the storage type;
it holds none of the layer's arithmetic, so both the HIP path (tests, bench)
and the float64 oracle consume exactly the same values.

Every tensor gets its own PCG64 stream, spawned from SeedSequence(seed) in a
fixed order, so a tensor's values do not depend on the sizes of the others.
Distributions (the layer-shaped synthetic recipe):

    q, k, v raw projections ~ N(0, 1)
    conv taps               ~ N(0, 0.5^2)
    beta                    = sigmoid(N(0, 1))
    gate pre-activation f   ~ N(0, 1)
    A_log                   ~ U(0, ln 16) per head         (fp32)
    dt_bias                 ~ N(0, 0.1^2) per channel      (fp32)
    gate_lower_bound        = -5
    output-gate logits      ~ N(0, 1)
    RMSNorm weight          ~ U(0.5, 1.5)
    query scale             = d_k^-1/2

bf16 workloads round every io tensor to bf16 (round-to-nearest-even from
fp32); A_log and dt_bias stay fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np

STREAMS = ("qkv", "conv_w", "f", "dt_bias", "A_log", "beta", "g_out", "norm_w", "accepted")


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    W: int
    chunk: int
    io: str            # "f32" or "bf16"
    seed: int
    prefix_T: int = 0  # tokens run before the step under test (pre-filled state)
    splits: int = 1    # number of chained calls the T tokens are split into
    lb: float = -5.0
    gate: str = "sigmoid"  # "sigmoid" (bounded by lb) or "softplus" (no bound: lb is absent, NaN)

    @property
    def c_qkv(self) -> int:
        return 2 * self.H * self.dk + self.H * self.dv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny layer, fp32 io: parity at 1e-5.
    "tiny_fp32": Workload("tiny_fp32", B=1, T=64, H=2, dk=16, dv=16, W=4, chunk=16, io="f32", seed=0),
    # One decode step over 64 sequences whose states were pre-filled by 256 tokens.
    "decode_b64": Workload("decode_b64", B=64, T=1, H=32, dk=128, dv=128, W=4, chunk=64, io="bf16",
                           seed=1, prefix_T=256),
    # Chunked prefill of one 4096-token sequence from zero state.
    "prefill_t4096": Workload("prefill_t4096", B=1, T=4096, H=32, dk=128, dv=128, W=4, chunk=64,
                              io="bf16", seed=2),
    # 32768 tokens as 8 chained calls of 4096 that carry state and conv state.
    "long_prefill_t32768": Workload("long_prefill_t32768", B=1, T=32768, H=32, dk=128, dv=128, W=4,
                                    chunk=64, io="bf16", seed=3, splits=8),
    # Speculative verify of 8 draft tokens on 16 sequences pre-filled by 2048 tokens.
    "verify_b16": Workload("verify_b16", B=16, T=8, H=32, dk=128, dv=128, W=4, chunk=64, io="bf16",
                           seed=4, prefix_T=2048),
}


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the fp32 values they represent (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_io(x: np.ndarray, io: str) -> np.ndarray:
    """Round an array to the io storage type; returns fp32 values."""
    x = np.asarray(x, dtype=np.float32)
    if io == "f32":
        return np.ascontiguousarray(x)
    if io == "bf16":
        return bf16_bits_to_f32(bf16_bits(x))
    raise ValueError(io)


def _rngs(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(STREAMS, children)}


def _normal(rng, shape, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _sigmoid_of_normal(rng, shape) -> np.ndarray:
    z = rng.standard_normal(size=shape).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def generate(wl: Workload) -> dict:
    """All inputs of a workload as fp32 numpy arrays holding io-type values.

    Token tensors cover prefix_T + T tokens along axis 1; the first prefix_T
    tokens are the ones that pre-fill the state, the rest are the call(s)
    under test.  Keys: qkv, f, beta, g_out [B, prefix_T+T, ...], conv_w,
    A_log, dt_bias, norm_w, lb, scale, accepted [B] (draft tokens accepted,
    uniform on 0..T), and zero initial state / conv state.
    """
    r = _rngs(wl.seed)
    io = wl.io
    B, H, dk, dv, W = wl.B, wl.H, wl.dk, wl.dv, wl.W
    TT = wl.prefix_T + wl.T
    out = {
        "qkv": round_to_io(_normal(r["qkv"], (B, TT, wl.c_qkv)), io),
        "conv_w": round_to_io(_normal(r["conv_w"], (wl.c_qkv, W), 0.5), io),
        "f": round_to_io(_normal(r["f"], (B, TT, H * dk)), io),
        "dt_bias": _normal(r["dt_bias"], (H * dk,), 0.1),
        "A_log": (r["A_log"].random(size=(H,), dtype=np.float32) * np.float32(math.log(16.0))),
        "beta": round_to_io(_sigmoid_of_normal(r["beta"], (B, TT, H)), io),
        "g_out": round_to_io(_normal(r["g_out"], (B, TT, H * dv)), io),
        "norm_w": round_to_io(r["norm_w"].random(size=(dv,), dtype=np.float32) + np.float32(0.5), io),
        "accepted": r["accepted"].integers(0, wl.T + 1, size=(B,)).astype(np.int32),
        "lb": float(wl.lb) if wl.gate == "sigmoid" else float("nan"),
        "gate": wl.gate,
        "scale": float(dk) ** -0.5,
        "state0": np.zeros((B, H, dk, dv), dtype=np.float32),
        "conv_state0": np.zeros((B, wl.c_qkv, W - 1), dtype=np.float32),
    }
    return out


def split_tokens(inp: dict, t0: int, t1: int) -> dict:
    """The token tensors restricted to tokens [t0, t1) (views)."""
    return {k: inp[k][:, t0:t1] for k in ("qkv", "f", "beta", "g_out")}


def select_heads(wl: Workload, inp: dict, heads) -> tuple:
    """Restrict a workload's inputs to a subset of heads.

    Heads are independent in this layer (own conv channels, own gate
    channels, own state), so a subset of heads is a smaller layer of the
    same kind.  Returns (workload with H = len(heads), inputs).
    """
    heads = list(heads)
    H, dk, dv = wl.H, wl.dk, wl.dv
    qc = np.concatenate([np.arange(h * dk, (h + 1) * dk) for h in heads])
    kc = qc + H * dk
    vc = np.concatenate([2 * H * dk + np.arange(h * dv, (h + 1) * dv) for h in heads])
    ch = np.concatenate([qc, kc, vc])
    fc = qc
    oc = np.concatenate([np.arange(h * dv, (h + 1) * dv) for h in heads])
    sub = dict(inp)
    sub["qkv"] = inp["qkv"][..., ch]
    sub["conv_w"] = inp["conv_w"][ch]
    sub["f"] = inp["f"][..., fc]
    sub["dt_bias"] = inp["dt_bias"][fc]
    sub["A_log"] = inp["A_log"][heads]
    sub["beta"] = inp["beta"][..., heads]
    sub["g_out"] = inp["g_out"][..., oc]
    sub["state0"] = inp["state0"][:, heads]
    sub["conv_state0"] = inp["conv_state0"][:, ch]
    return wl.with_(H=len(heads)), sub


def varlen_lengths(total: int, n: int, seed: int, zeros: int = 0) -> list:
    """n sequence lengths summing to `total`, for packed variable-length calls: a seeded
    log-normal mix (spread of about 4x between short and long sequences), `zeros` of them
    empty, rounded so that the sum is exact."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    w = rng.lognormal(mean=0.0, sigma=0.7, size=n)
    w[:zeros] = 0.0
    rng.shuffle(w)
    raw = w / w.sum() * total
    lens = np.floor(raw).astype(np.int64)
    rest = total - int(lens.sum())
    order = np.argsort(-(raw - lens))
    for i in order[:rest]:
        lens[i] += 1
    return [int(x) for x in lens]


def cu_seqlens(lengths) -> list:
    """Packed offsets [0, l0, l0+l1, ...] of a list of sequence lengths."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


@dataclass(frozen=True)
class ProjWorkload:
    name: str
    T: int
    hidden: int
    H: int
    d: int
    rank: int
    seed: int


PROJ_WORKLOADS = {
    # the input projection ahead of prefill_t4096: 4096 tokens of a 4096-wide model (the pages give
    # no model width; 4096 = H*d is the reading taken), H=32, d=128, f/g rank 128
    "projection_t4096": ProjWorkload("projection_t4096", T=4096, hidden=4096, H=32, d=128, rank=128, seed=6),
}


def generate_projection(wl: ProjWorkload) -> dict:
    """Hidden states x ~ N(0, 1) and Linear weights ~ N(0, 1/in_features), all rounded to bf16
    (so the projected q, k, v, f and gate logits come out near N(0, 1), as in the layer's own
    synthetic inputs).  Keys: x [T, hidden], w_in [3Hd + 2r + H, hidden], w_fb, w_gb [Hd, r]."""
    children = np.random.SeedSequence(wl.seed).spawn(4)
    r = [np.random.Generator(np.random.PCG64(c)) for c in children]
    HD = wl.H * wl.d
    n = 3 * HD + 2 * wl.rank + wl.H
    return {
        "x": round_to_io(_normal(r[0], (wl.T, wl.hidden)), "bf16"),
        "w_in": round_to_io(_normal(r[1], (n, wl.hidden), wl.hidden ** -0.5), "bf16"),
        "w_fb": round_to_io(_normal(r[2], (HD, wl.rank), wl.rank ** -0.5), "bf16"),
        "w_gb": round_to_io(_normal(r[3], (HD, wl.rank), wl.rank ** -0.5), "bf16"),
    }
