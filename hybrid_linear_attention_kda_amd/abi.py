"""ctypes binding over libkda.so, the C ABI declared in include/kda.h.

Argument marshalling only: torch supplies device memory and the stream,
every step of the layer runs in the library's HIP kernels.  Tensor shapes
and dtypes are checked here before a pointer is handed to the library (the
C side cannot see shapes), so a wrongly sized buffer raises instead of
reaching a kernel.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import c_float, c_int32, c_size_t, c_void_p
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY names another build of the same library (the host-sanitizer build of
# build.build_host_sanitized); by default the in-tree libkda.so is loaded.
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(HERE, "libkda.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kda.h")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_HIP = 0, 1, 2, 3
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_BOUNDED_SIGMOID, KDA_GATE_SOFTPLUS = 0, 1
_TORCH_OF = {KDA_F32: torch.float32, KDA_BF16: torch.bfloat16}


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"KDA status {status}: {message}")
        self.status = status


class KdaLayerDesc(ctypes.Structure):
    _fields_ = [
        ("num_heads", c_int32), ("head_dim_k", c_int32), ("head_dim_v", c_int32), ("conv_width", c_int32),
        ("chunk_size", c_int32), ("io_dtype", c_int32), ("out_dtype", c_int32),
        ("gate_lower_bound", c_float), ("l2_eps", c_float), ("rms_eps", c_float), ("scale", c_float),
        ("conv_w", c_void_p), ("A_log", c_void_p), ("dt_bias", c_void_p), ("norm_w", c_void_p),
        ("gate_kind", c_int32),
    ]


class KdaProjDesc(ctypes.Structure):
    _fields_ = [
        ("num_heads", c_int32), ("head_dim", c_int32), ("hidden", c_int32), ("rank", c_int32),
        ("out_dtype", c_int32), ("w_in", c_void_p), ("w_fb", c_void_p), ("w_gb", c_void_p),
    ]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libkda.so (built in-tree by the package's build step)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -m hybrid_linear_attention_kda_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    P = c_void_p
    D = ctypes.POINTER(KdaLayerDesc)
    sigs = {
        "kda_abi_version": (c_int32, []),
        "kda_status_string": (ctypes.c_char_p, [c_int32]),
        "kda_last_error": (ctypes.c_char_p, []),
        "kda_prefill_workspace_size": (c_size_t, [D, c_int32, c_int32]),
        "kda_prefill": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P, P, P, c_size_t, P]),
        "kda_prefill_noalloc": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P, P, P]),
        "kda_decode_step": (c_int32, [D, c_int32, P, P, P, P, P, P, P, P]),
        "kda_verify_block": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P, P, P, P]),
        "kda_rollback": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P]),
        "kda_verify_tape_size": (c_size_t, [D, c_int32, c_int32]),
        "kda_prefill_varlen_workspace_size": (c_size_t, [D, c_int32, P]),
        "kda_input_projection_workspace_size": (c_size_t, [ctypes.POINTER(KdaProjDesc), c_int32]),
        "kda_input_projection": (c_int32, [ctypes.POINTER(KdaProjDesc), c_int32, P, P, P, P, P, P, c_size_t, P]),
        "kda_prefill_varlen": (c_int32, [D, c_int32, P, P, c_int32, P, P, P, P, P, P, P, P, c_size_t, P]),
        "kda_verify_block_tape": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P, P, P, P]),
        "kda_commit_tape": (c_int32, [D, c_int32, c_int32, P, P, P, P, P, P]),
        "kda_timing_enable": (c_int32, [c_int32]),
        "kda_timing_read": (c_int32, [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(c_float), c_int32]),
        "kda_measure_stream": (c_int32, [P, P, c_size_t, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions include/kda.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(kda_[a-z_0-9]+)\s*\(", text, re.M)))


def _check(status: int):
    if status != KDA_OK:
        msg = load().kda_last_error().decode()
        raise KdaError(status, msg)


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class KdaLayer:
    """A layer description plus the device parameter tensors it points to."""
    H: int
    D: int
    W: int
    chunk: int
    io_dtype: int
    out_dtype: int
    lb: float
    scale: float
    conv_w: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    norm_w: torch.Tensor
    l2_eps: float = 1e-6
    rms_eps: float = 1e-5
    gate_kind: int = 0  # KDA_GATE_BOUNDED_SIGMOID; KDA_GATE_SOFTPLUS (1) takes lb = NaN

    def __post_init__(self):
        io = _TORCH_OF[self.io_dtype]
        c = 3 * self.H * self.D
        _expect(self.conv_w, (c, self.W), io, "conv_w")
        _expect(self.A_log, (self.H,), torch.float32, "A_log")
        _expect(self.dt_bias, (self.H * self.D,), torch.float32, "dt_bias")
        _expect(self.norm_w, (self.D,), io, "norm_w")
        self.desc = KdaLayerDesc(self.H, self.D, self.D, self.W, self.chunk, self.io_dtype, self.out_dtype,
                                 self.lb, self.l2_eps, self.rms_eps, self.scale, _ptr(self.conv_w),
                                 _ptr(self.A_log), _ptr(self.dt_bias), _ptr(self.norm_w), self.gate_kind)

    @property
    def c_qkv(self) -> int:
        return 3 * self.H * self.D

    @property
    def io_torch(self):
        return _TORCH_OF[self.io_dtype]

    @property
    def out_torch(self):
        return _TORCH_OF[self.out_dtype]


@dataclass
class KdaProjection:
    """An input-projection description plus its device weight tensors (Linear weights, [out, in])."""
    H: int
    D: int
    hidden: int
    rank: int
    out_dtype: int
    w_in: torch.Tensor  # [3*H*D + 2*rank + H, hidden] bf16
    w_fb: torch.Tensor  # [H*D, rank] bf16
    w_gb: torch.Tensor  # [H*D, rank] bf16

    def __post_init__(self):
        n = 3 * self.H * self.D + 2 * self.rank + self.H
        _expect(self.w_in, (n, self.hidden), torch.bfloat16, "w_in")
        _expect(self.w_fb, (self.H * self.D, self.rank), torch.bfloat16, "w_fb")
        _expect(self.w_gb, (self.H * self.D, self.rank), torch.bfloat16, "w_gb")
        self.desc = KdaProjDesc(self.H, self.D, self.hidden, self.rank, self.out_dtype, _ptr(self.w_in),
                                _ptr(self.w_fb), _ptr(self.w_gb))

    @property
    def out_torch(self):
        return _TORCH_OF[self.out_dtype]


def _expect(t, shape, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_tokens(layer: KdaLayer, B, T, qkv, f, beta, g_out):
    io = layer.io_torch
    _expect(qkv, (B, T, layer.c_qkv), io, "qkv")
    _expect(f, (B, T, layer.H * layer.D), io, "f")
    _expect(beta, (B, T, layer.H), io, "beta")
    _expect(g_out, (B, T, layer.H * layer.D), io, "g_out")


def _check_state(layer: KdaLayer, B, state, conv_state):
    _expect(state, (B, layer.H, layer.D, layer.D), torch.float32, "state")
    if layer.W > 1:
        _expect(conv_state, (B, layer.c_qkv, layer.W - 1), layer.io_torch, "conv_state")


def kda_prefill_workspace_size(layer: KdaLayer, B: int, T: int) -> int:
    n = load().kda_prefill_workspace_size(ctypes.byref(layer.desc), B, T)
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARGUMENT, load().kda_last_error().decode())
    return n


def kda_prefill(layer: KdaLayer, qkv, f, beta, g_out, state, conv_state, out, workspace=None, stream=None):
    B, T = qkv.shape[0], qkv.shape[1]
    _check_tokens(layer, B, T, qkv, f, beta, g_out)
    _check_state(layer, B, state, conv_state)
    _expect(out, (B, T, layer.H * layer.D), layer.out_torch, "out")
    need = kda_prefill_workspace_size(layer, B, T)
    ws_bytes = 0
    if workspace is not None:
        ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace of {ws_bytes} bytes, {need} needed")
    _check(load().kda_prefill(ctypes.byref(layer.desc), B, T, _ptr(qkv), _ptr(f), _ptr(beta), _ptr(g_out),
                              _ptr(state), _ptr(conv_state), _ptr(out), _ptr(workspace), ws_bytes,
                              _stream(stream)))


def kda_prefill_noalloc(layer: KdaLayer, qkv, f, beta, g_out, state, conv_state, out, stream=None):
    """kda_prefill with the library's fixed scratch instead of a caller workspace."""
    B, T = qkv.shape[0], qkv.shape[1]
    _check_tokens(layer, B, T, qkv, f, beta, g_out)
    _check_state(layer, B, state, conv_state)
    _expect(out, (B, T, layer.H * layer.D), layer.out_torch, "out")
    _check(load().kda_prefill_noalloc(ctypes.byref(layer.desc), B, T, _ptr(qkv), _ptr(f), _ptr(beta), _ptr(g_out),
                                      _ptr(state), _ptr(conv_state), _ptr(out), _stream(stream)))


def kda_decode_step(layer: KdaLayer, qkv, f, beta, g_out, state, conv_state, out, stream=None):
    B = qkv.shape[0]
    _check_tokens(layer, B, 1, qkv.view(B, 1, -1), f.view(B, 1, -1), beta.view(B, 1, -1), g_out.view(B, 1, -1))
    _check_state(layer, B, state, conv_state)
    _expect(out.view(B, 1, -1), (B, 1, layer.H * layer.D), layer.out_torch, "out")
    _check(load().kda_decode_step(ctypes.byref(layer.desc), B, _ptr(qkv), _ptr(f), _ptr(beta), _ptr(g_out),
                                  _ptr(state), _ptr(conv_state), _ptr(out), _stream(stream)))


def kda_verify_block(layer: KdaLayer, qkv, f, beta, g_out, state, conv_state, snaps, out, stream=None):
    B, T_d = qkv.shape[0], qkv.shape[1]
    _check_tokens(layer, B, T_d, qkv, f, beta, g_out)
    _check_state(layer, B, state, conv_state)
    _expect(snaps, (B, T_d, layer.H, layer.D, layer.D), torch.float32, "snaps")
    _expect(out, (B, T_d, layer.H * layer.D), layer.out_torch, "out")
    _check(load().kda_verify_block(ctypes.byref(layer.desc), B, T_d, _ptr(qkv), _ptr(f), _ptr(beta),
                                   _ptr(g_out), _ptr(state), _ptr(conv_state), _ptr(snaps), _ptr(out),
                                   _stream(stream)))


def kda_rollback(layer: KdaLayer, accepted, snaps, qkv_block, state, conv_state, stream=None):
    B, T_d = qkv_block.shape[0], qkv_block.shape[1]
    if len(accepted) != B:
        raise ValueError(f"accepted has {len(accepted)} entries, expected {B}")
    acc = (ctypes.c_int32 * B)(*[int(m) for m in accepted])
    _expect(qkv_block, (B, T_d, layer.c_qkv), layer.io_torch, "qkv_block")
    _expect(snaps, (B, T_d, layer.H, layer.D, layer.D), torch.float32, "snaps")
    _check_state(layer, B, state, conv_state)
    _check(load().kda_rollback(ctypes.byref(layer.desc), B, T_d, ctypes.cast(acc, c_void_p), _ptr(snaps),
                               _ptr(qkv_block), _ptr(state), _ptr(conv_state), _stream(stream)))


def _int32_array(values):
    vals = [int(v) for v in values]
    return (ctypes.c_int32 * max(len(vals), 1))(*vals), len(vals)


def kda_prefill_varlen_workspace_size(layer: KdaLayer, cu_seqlens) -> int:
    cu, n = _int32_array(cu_seqlens)
    size = load().kda_prefill_varlen_workspace_size(ctypes.byref(layer.desc), n - 1, ctypes.cast(cu, c_void_p))
    if size == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARGUMENT, load().kda_last_error().decode())
    return size


def kda_prefill_varlen(layer: KdaLayer, cu_seqlens, slots, qkv, f, beta, g_out, state, conv_state, out,
                       workspace=None, stream=None):
    """Sequences packed along the token axis (cu_seqlens, host list of N+1 offsets), each continuing
    the state in its own slot (slots: host list of N, or None for slot i)."""
    cu, n1 = _int32_array(cu_seqlens)
    N = n1 - 1
    total = int(cu_seqlens[-1]) if N >= 0 else 0
    num_slots = state.shape[0]
    sl = None
    if slots is not None:
        if len(slots) != N:
            raise ValueError(f"slots has {len(slots)} entries, expected {N}")
        sl, _ = _int32_array(slots)
    _check_tokens(layer, 1, total, qkv.view(1, total, -1), f.view(1, total, -1), beta.view(1, total, -1),
                  g_out.view(1, total, -1))
    _check_state(layer, num_slots, state, conv_state)
    _expect(out.view(1, total, -1), (1, total, layer.H * layer.D), layer.out_torch, "out")
    need = kda_prefill_varlen_workspace_size(layer, cu_seqlens)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace of {ws_bytes} bytes, {need} needed")
    _check(load().kda_prefill_varlen(ctypes.byref(layer.desc), N, ctypes.cast(cu, c_void_p),
                                     ctypes.cast(sl, c_void_p) if sl is not None else None, num_slots,
                                     _ptr(qkv), _ptr(f), _ptr(beta), _ptr(g_out), _ptr(state), _ptr(conv_state),
                                     _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def kda_input_projection_workspace_size(proj: KdaProjection, T: int) -> int:
    n = load().kda_input_projection_workspace_size(ctypes.byref(proj.desc), T)
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARGUMENT, load().kda_last_error().decode())
    return n


def kda_input_projection(proj: KdaProjection, x, qkv, f, beta, g_out, workspace, stream=None):
    """x [T, hidden] bf16 -> qkv [T, 3*H*D], f [T, H*D], beta [T, H], g_out [T, H*D]."""
    T = x.shape[0]
    _expect(x, (T, proj.hidden), torch.bfloat16, "x")
    ot = proj.out_torch
    HD = proj.H * proj.D
    _expect(qkv, (T, 3 * HD), ot, "qkv")
    _expect(f, (T, HD), ot, "f")
    _expect(beta, (T, proj.H), ot, "beta")
    _expect(g_out, (T, HD), ot, "g_out")
    need = kda_input_projection_workspace_size(proj, T)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace of {ws_bytes} bytes, {need} needed")
    _check(load().kda_input_projection(ctypes.byref(proj.desc), T, _ptr(x), _ptr(qkv), _ptr(f), _ptr(beta),
                                       _ptr(g_out), _ptr(workspace), ws_bytes, _stream(stream)))


def kda_verify_tape_size(layer: KdaLayer, B: int, T_d: int) -> int:
    n = load().kda_verify_tape_size(ctypes.byref(layer.desc), B, T_d)
    if n == ctypes.c_size_t(-1).value:
        raise KdaError(KDA_ERR_INVALID_ARGUMENT, load().kda_last_error().decode())
    return n


def kda_verify_block_tape(layer: KdaLayer, qkv, f, beta, g_out, state, conv_state, tape, out, stream=None):
    B, T_d = qkv.shape[0], qkv.shape[1]
    _check_tokens(layer, B, T_d, qkv, f, beta, g_out)
    _check_state(layer, B, state, conv_state)
    _expect(tape, (B, T_d, layer.H, 3, layer.D), torch.float32, "tape")
    _expect(out, (B, T_d, layer.H * layer.D), layer.out_torch, "out")
    _check(load().kda_verify_block_tape(ctypes.byref(layer.desc), B, T_d, _ptr(qkv), _ptr(f), _ptr(beta),
                                        _ptr(g_out), _ptr(state), _ptr(conv_state), _ptr(tape), _ptr(out),
                                        _stream(stream)))


def kda_commit_tape(layer: KdaLayer, accepted, tape, qkv_block, state, conv_state, stream=None):
    B, T_d = qkv_block.shape[0], qkv_block.shape[1]
    if len(accepted) != B:
        raise ValueError(f"accepted has {len(accepted)} entries, expected {B}")
    acc = (ctypes.c_int32 * B)(*[int(m) for m in accepted])
    _expect(qkv_block, (B, T_d, layer.c_qkv), layer.io_torch, "qkv_block")
    _expect(tape, (B, T_d, layer.H, 3, layer.D), torch.float32, "tape")
    _check_state(layer, B, state, conv_state)
    _check(load().kda_commit_tape(ctypes.byref(layer.desc), B, T_d, ctypes.cast(acc, c_void_p), _ptr(tape),
                                  _ptr(qkv_block), _ptr(state), _ptr(conv_state), _stream(stream)))


def timing_enable(on: bool) -> bool:
    """Per-kernel timing of later calls on this thread (kda_timing_enable); returns the old setting."""
    return bool(load().kda_timing_enable(1 if on else 0))


def timing_read(cap: int = 1 << 16) -> list:
    """(kernel name, milliseconds) of every kernel launched since timing was enabled or last read,
    in launch order (kda_timing_read); waits for those kernels."""
    names = (ctypes.c_char_p * cap)()
    ms = (c_float * cap)()
    n = load().kda_timing_read(names, ms, cap)
    if n < 0:
        raise KdaError(KDA_ERR_HIP, load().kda_last_error().decode())
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


def measure_stream(dst, src=None, stream=None):
    """The library's streaming copy of src into dst (kda_measure_stream; src None: a zero fill of
    dst), for measuring HBM ceilings: contiguous device tensors, the byte size of dst."""
    nbytes = dst.numel() * dst.element_size()
    if src is not None and src.numel() * src.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    _check(load().kda_measure_stream(_ptr(dst), None if src is None else _ptr(src), nbytes, _stream(stream)))
