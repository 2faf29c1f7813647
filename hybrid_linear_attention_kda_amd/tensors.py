"""Host arrays -> device tensors for the library calls (marshalling only).

The seeded generators produce fp32 numpy arrays whose values are exactly
representable in the io type; here they become torch tensors of that type on
the target device, bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

from . import abi
from .inputs import Workload, bf16_bits


def to_device(x: np.ndarray, io: str, device) -> torch.Tensor:
    if io == "bf16":
        bits = np.ascontiguousarray(bf16_bits(x)).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    if io == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    raise ValueError(io)


def io_code(io: str) -> int:
    return abi.KDA_BF16 if io == "bf16" else abi.KDA_F32


def make_layer(wl: Workload, inp: dict, device, out: str = "f32", chunk: int = None) -> abi.KdaLayer:
    """A KdaLayer whose parameters are the workload's, on `device`."""
    return abi.KdaLayer(
        H=wl.H, D=wl.dk, W=wl.W, chunk=chunk or wl.chunk, io_dtype=io_code(wl.io), out_dtype=io_code(out),
        lb=inp["lb"], scale=inp["scale"], gate_kind={"sigmoid": 0, "softplus": 1}[inp.get("gate", "sigmoid")],
        rms_eps=inp.get("rms_eps", 1e-5),
        conv_w=to_device(inp["conv_w"], wl.io, device),
        A_log=torch.from_numpy(np.ascontiguousarray(inp["A_log"], dtype=np.float32)).to(device),
        dt_bias=torch.from_numpy(np.ascontiguousarray(inp["dt_bias"], dtype=np.float32)).to(device),
        norm_w=to_device(inp["norm_w"], wl.io, device),
    )


def token_tensors(wl: Workload, inp: dict, t0: int, t1: int, device) -> dict:
    """qkv, f, beta, g_out for tokens [t0, t1) of every sequence, on `device`."""
    return {k: to_device(inp[k][:, t0:t1], wl.io, device) for k in ("qkv", "f", "beta", "g_out")}


def to_host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()
