"""Host-side checks of the C ABI: the library loads, exports what include/kda.h
declares, and refuses bad arguments before touching any device memory.

No call here reaches a kernel: every case fails validation (or is an empty
no-op), which happens before the first HIP call, so these run without a GPU.
"""
import ctypes
import math

import pytest

from hybrid_linear_attention_kda_amd import abi

FAKE = 0x10000  # aligned, never dereferenced: validation fails or returns before any launch


def desc(**kw):
    d = dict(num_heads=2, head_dim_k=16, head_dim_v=16, conv_width=4, chunk_size=16, io_dtype=0, out_dtype=0,
             gate_lower_bound=-5.0, l2_eps=1e-6, rms_eps=1e-5, scale=0.25, conv_w=FAKE, A_log=FAKE,
             dt_bias=FAKE, norm_w=FAKE, gate_kind=0)
    d.update(kw)
    return abi.KdaLayerDesc(*[d[n] for n, _ in abi.KdaLayerDesc._fields_])


def prefill(d, B=1, T=8, ptr=FAKE, ws=0, ws_bytes=0):
    lib = abi.load()
    return lib.kda_prefill(ctypes.byref(d) if d is not None else None, B, T, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                           ws, ws_bytes, None)


def test_library_exports_every_header_function():
    lib = abi.load()
    names = abi.header_functions()
    assert set(names) == {"kda_abi_version", "kda_status_string", "kda_last_error", "kda_prefill_workspace_size",
                          "kda_prefill", "kda_decode_step", "kda_verify_block", "kda_rollback",
                          "kda_verify_tape_size", "kda_verify_block_tape", "kda_commit_tape",
                          "kda_prefill_varlen_workspace_size", "kda_prefill_varlen",
                          "kda_input_projection_workspace_size", "kda_input_projection",
                          "kda_timing_enable", "kda_timing_read", "kda_prefill_noalloc", "kda_measure_stream"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kda_abi_version() == 3
    assert lib.kda_status_string(0) == b"ok"


@pytest.mark.parametrize("kw,status,needle", [
    (dict(gate_lower_bound=math.nan), abi.KDA_ERR_INVALID_ARGUMENT, b"gate_lower_bound is absent"),
    (dict(gate_lower_bound=math.inf), abi.KDA_ERR_INVALID_ARGUMENT, b"not finite"),
    # the softplus branch is the one without a bound: a finite bound with it is an error, and so is
    # a gate kind the header does not define
    (dict(gate_kind=1), abi.KDA_ERR_INVALID_ARGUMENT, b"must be NaN"),
    (dict(gate_kind=1, gate_lower_bound=math.inf), abi.KDA_ERR_INVALID_ARGUMENT, b"must be NaN"),
    (dict(gate_kind=2), abi.KDA_ERR_INVALID_ARGUMENT, b"not a kda_gate_kind"),
    (dict(gate_kind=-1, gate_lower_bound=math.nan), abi.KDA_ERR_INVALID_ARGUMENT, b"not a kda_gate_kind"),
    (dict(head_dim_v=8), abi.KDA_ERR_UNSUPPORTED, b"head_dim_k"),
    (dict(head_dim_k=48, head_dim_v=48), abi.KDA_ERR_UNSUPPORTED, b"head dim 48"),
    (dict(conv_width=9), abi.KDA_ERR_UNSUPPORTED, b"conv_width"),
    (dict(conv_width=0), abi.KDA_ERR_INVALID_ARGUMENT, b"conv_width"),
    (dict(chunk_size=128), abi.KDA_ERR_UNSUPPORTED, b"chunk_size"),
    (dict(chunk_size=0), abi.KDA_ERR_INVALID_ARGUMENT, b"chunk_size"),
    (dict(io_dtype=7), abi.KDA_ERR_INVALID_ARGUMENT, b"io_dtype"),
    (dict(l2_eps=0.0), abi.KDA_ERR_INVALID_ARGUMENT, b"l2_eps"),
    (dict(rms_eps=-1.0), abi.KDA_ERR_INVALID_ARGUMENT, b"rms_eps"),
    (dict(num_heads=0), abi.KDA_ERR_INVALID_ARGUMENT, b"num_heads"),
    (dict(A_log=0), abi.KDA_ERR_INVALID_ARGUMENT, b"desc.A_log is null"),
    (dict(conv_w=FAKE + 4), abi.KDA_ERR_INVALID_ARGUMENT, b"not 16-byte aligned"),
])
def test_prefill_rejects_bad_descriptor(kw, status, needle):
    assert prefill(desc(**kw)) == status
    assert needle in abi.load().kda_last_error()


def test_softplus_descriptor_passes_validation():
    # a NaN bound with the softplus kind passes validation; B = 0 leaves nothing to launch
    assert prefill(desc(gate_kind=1, gate_lower_bound=math.nan), B=0) == abi.KDA_OK


def test_null_descriptor_and_bad_sizes():
    lib = abi.load()
    assert prefill(None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert prefill(desc(), B=-1) == abi.KDA_ERR_INVALID_ARGUMENT
    assert prefill(desc(), B=70000) == abi.KDA_ERR_UNSUPPORTED
    assert prefill(desc(), ptr=0) == abi.KDA_ERR_INVALID_ARGUMENT
    assert prefill(desc(), ptr=FAKE + 2) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"not 16-byte aligned" in lib.kda_last_error()
    # one call indexes token-heads with 32-bit integers: 2 heads x 2^30 tokens is refused up front
    assert prefill(desc(), B=1, T=(1 << 30)) == abi.KDA_ERR_UNSUPPORTED
    assert b"token-heads" in lib.kda_last_error()


def test_empty_calls_are_no_ops():
    # B = 0 or T = 0: nothing to do, no pointer is looked at and no kernel runs.
    assert prefill(desc(), B=0, ptr=0) == abi.KDA_OK
    assert prefill(desc(), T=0, ptr=0) == abi.KDA_OK
    lib = abi.load()
    d = desc()
    assert lib.kda_decode_step(ctypes.byref(d), 0, 0, 0, 0, 0, 0, 0, 0, None) == abi.KDA_OK
    assert lib.kda_verify_block(ctypes.byref(d), 3, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == abi.KDA_OK
    acc = (ctypes.c_int32 * 2)(0, 0)  # nothing accepted: no-op
    assert lib.kda_rollback(ctypes.byref(d), 2, 8, ctypes.cast(acc, ctypes.c_void_p), 0, 0, 0, 0, None) == abi.KDA_OK


def test_verify_and_rollback_validation():
    lib = abi.load()
    d = desc()
    P = FAKE
    assert lib.kda_verify_block(ctypes.byref(d), 1, 256, P, P, P, P, P, P, P, P, None) == abi.KDA_ERR_UNSUPPORTED
    assert lib.kda_verify_block(ctypes.byref(d), 1, 8, P, P, P, P, P, P, 0, P, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"snaps is null" in lib.kda_last_error()
    for bad in (-1, 9):
        acc = (ctypes.c_int32 * 2)(3, bad)
        st = lib.kda_rollback(ctypes.byref(d), 2, 8, ctypes.cast(acc, ctypes.c_void_p), P, P, P, P, None)
        assert st == abi.KDA_ERR_INVALID_ARGUMENT
        assert f"accepted[1] = {bad} outside 0..8".encode() in lib.kda_last_error()
    assert lib.kda_rollback(ctypes.byref(d), 2, 8, None, P, P, P, P, None) == abi.KDA_ERR_INVALID_ARGUMENT


def test_verify_tape_and_commit_validation():
    lib = abi.load()
    d = desc()
    P = FAKE
    assert lib.kda_verify_block_tape(ctypes.byref(d), 3, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == abi.KDA_OK
    assert lib.kda_verify_block_tape(ctypes.byref(d), 1, 256, P, P, P, P, P, P, P, P, None) == abi.KDA_ERR_UNSUPPORTED
    assert lib.kda_verify_block_tape(ctypes.byref(d), 1, 8, P, P, P, P, P, P, 0, P, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"tape is null" in lib.kda_last_error()
    acc = (ctypes.c_int32 * 2)(0, 0)  # nothing accepted: no-op, no pointer looked at
    assert lib.kda_commit_tape(ctypes.byref(d), 2, 8, ctypes.cast(acc, ctypes.c_void_p), 0, 0, 0, 0, None) == abi.KDA_OK
    for bad in (-1, 9):
        acc = (ctypes.c_int32 * 2)(3, bad)
        st = lib.kda_commit_tape(ctypes.byref(d), 2, 8, ctypes.cast(acc, ctypes.c_void_p), P, P, P, P, None)
        assert st == abi.KDA_ERR_INVALID_ARGUMENT
        assert f"accepted[1] = {bad} outside 0..8".encode() in lib.kda_last_error()
    acc = (ctypes.c_int32 * 2)(3, 0)
    st = lib.kda_commit_tape(ctypes.byref(d), 2, 8, ctypes.cast(acc, ctypes.c_void_p), 0, P, P, P, None)
    assert st == abi.KDA_ERR_INVALID_ARGUMENT and b"tape is null" in lib.kda_last_error()
    # B * T_d * H * 3 * d fp32 (the test descriptor: H = 2, d = 16)
    assert lib.kda_verify_tape_size(ctypes.byref(d), 4, 8) == 4 * 8 * d.num_heads * 3 * d.head_dim_k * 4
    bad = desc(gate_lower_bound=math.nan)
    assert lib.kda_verify_tape_size(ctypes.byref(bad), 4, 8) == ctypes.c_size_t(-1).value


def test_draft_block_limit_is_refused_by_every_call():
    # T_d <= 255 is the documented limit of the verify, rollback, tape and commit calls and of the
    # tape-size query; T_d = 256 is refused up front with KDA_ERR_UNSUPPORTED, never clamped
    lib = abi.load()
    d = desc()
    P = FAKE
    acc = (ctypes.c_int32 * 1)(3)
    accp = ctypes.cast(acc, ctypes.c_void_p)
    calls = {
        "kda_verify_block": lambda T_d: lib.kda_verify_block(ctypes.byref(d), 1, T_d, P, P, P, P, P, P, P, P, None),
        "kda_verify_block_tape": lambda T_d: lib.kda_verify_block_tape(ctypes.byref(d), 1, T_d, P, P, P, P, P, P, P, P,
                                                                       None),
        "kda_rollback": lambda T_d: lib.kda_rollback(ctypes.byref(d), 1, T_d, accp, P, P, P, P, None),
        "kda_commit_tape": lambda T_d: lib.kda_commit_tape(ctypes.byref(d), 1, T_d, accp, P, P, P, P, None),
    }
    for name, call in calls.items():
        assert call(256) == abi.KDA_ERR_UNSUPPORTED, name
        assert b"T_d = 256 > 255" in lib.kda_last_error(), name
    assert lib.kda_verify_tape_size(ctypes.byref(d), 2, 256) == ctypes.c_size_t(-1).value
    assert b"T_d = 256 > 255" in lib.kda_last_error()
    # the largest block is sized exactly: B * T_d * H * 3 * d fp32
    assert lib.kda_verify_tape_size(ctypes.byref(d), 2, 255) == 2 * 255 * 2 * 3 * 16 * 4
    assert lib.kda_verify_tape_size(ctypes.byref(d), 0, 8) == 0
    assert lib.kda_verify_tape_size(ctypes.byref(d), -1, 8) == ctypes.c_size_t(-1).value


def test_varlen_validation_and_workspace_size():
    lib = abi.load()
    d = desc()
    P = FAKE

    def call(cu, slots=None, num_slots=4, ptr=P):
        c = (ctypes.c_int32 * len(cu))(*cu)
        sl = (ctypes.c_int32 * len(slots))(*slots) if slots is not None else None
        return lib.kda_prefill_varlen(ctypes.byref(d), len(cu) - 1, ctypes.cast(c, ctypes.c_void_p),
                                      ctypes.cast(sl, ctypes.c_void_p) if sl is not None else None, num_slots,
                                      ptr, ptr, ptr, ptr, ptr, ptr, ptr, 0, 0, None)

    assert lib.kda_prefill_varlen(ctypes.byref(d), 0, None, None, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, None) == abi.KDA_OK
    assert call([0, 0, 0], ptr=0) == abi.KDA_OK  # every sequence empty: nothing runs, no pointer looked at
    assert call([1, 3]) == abi.KDA_ERR_INVALID_ARGUMENT and b"cu_seqlens[0]" in lib.kda_last_error()
    assert call([0, 4, 2]) == abi.KDA_ERR_INVALID_ARGUMENT and b"decreases" in lib.kda_last_error()
    assert call([0, 2, 4], [1, 1]) == abi.KDA_ERR_INVALID_ARGUMENT and b"used by two" in lib.kda_last_error()
    assert call([0, 2, 4], [0, 4]) == abi.KDA_ERR_INVALID_ARGUMENT and b"outside 0..3" in lib.kda_last_error()
    assert call([0, 2, 4], num_slots=0) == abi.KDA_ERR_INVALID_ARGUMENT
    assert call([0, 2, 4], ptr=0) == abi.KDA_ERR_INVALID_ARGUMENT  # non-empty: pointers are checked
    assert call([0, 1 << 30]) == abi.KDA_ERR_UNSUPPORTED and b"token-heads" in lib.kda_last_error()
    c = (ctypes.c_int32 * 3)(0, 2, 4)
    assert lib.kda_prefill_varlen_workspace_size(ctypes.byref(d), 2, ctypes.cast(c, ctypes.c_void_p)) == 0  # fp32 path
    bad = (ctypes.c_int32 * 3)(0, 4, 2)
    assert lib.kda_prefill_varlen_workspace_size(ctypes.byref(d), 2, ctypes.cast(bad, ctypes.c_void_p)) == \
        ctypes.c_size_t(-1).value


def test_input_projection_validation():
    lib = abi.load()
    P = FAKE

    def pd(**kw):
        v = dict(num_heads=32, head_dim=128, hidden=4096, rank=128, out_dtype=abi.KDA_BF16, w_in=P, w_fb=P, w_gb=P)
        v.update(kw)
        return abi.KdaProjDesc(**v)

    def call(d, T=16, ptr=P, ws=0):
        return lib.kda_input_projection(ctypes.byref(d), T, ptr, ptr, ptr, ptr, ptr, ws, 1 << 30, None)

    assert call(pd(), T=0, ptr=0) == abi.KDA_OK
    assert call(pd(rank=64)) == abi.KDA_ERR_UNSUPPORTED and b"rank 64" in lib.kda_last_error()
    assert call(pd(num_heads=3, head_dim=16)) == abi.KDA_ERR_UNSUPPORTED
    assert call(pd(hidden=4100)) == abi.KDA_ERR_UNSUPPORTED
    assert call(pd(hidden=4160)) == abi.KDA_ERR_UNSUPPORTED and b"multiple of 128" in lib.kda_last_error()
    assert call(pd(hidden=1 << 17)) == abi.KDA_ERR_UNSUPPORTED
    assert call(pd(num_heads=1024, head_dim=128)) == abi.KDA_ERR_UNSUPPORTED
    assert call(pd(), T=(1 << 26)) == abi.KDA_ERR_UNSUPPORTED and b"token-heads" in lib.kda_last_error()
    assert call(pd(w_fb=0)) == abi.KDA_ERR_INVALID_ARGUMENT and b"desc.w_fb is null" in lib.kda_last_error()
    assert call(pd(out_dtype=5)) == abi.KDA_ERR_INVALID_ARGUMENT
    assert call(pd()) == abi.KDA_ERR_INVALID_ARGUMENT and b"workspace is null" in lib.kda_last_error()
    need = lib.kda_input_projection_workspace_size(ctypes.byref(pd()), 4096)
    act = (4096 * (2 * 128 + 32) * 4 + 255) // 256 * 256  # the rank / beta activations in fp32
    assert need == 9 * act  # ... and 8 K-piece partial sums of them
    # an odd 2r + H pads each partial-sum row to a multiple of 4 floats
    pitch = (4 * (2 * 128 + 1) + 15) // 16 * 16
    assert lib.kda_input_projection_workspace_size(ctypes.byref(pd(num_heads=1, head_dim=128)), 100) == \
        9 * ((100 * pitch + 255) // 256 * 256)
    assert lib.kda_input_projection_workspace_size(ctypes.byref(pd(rank=3)), 16) == ctypes.c_size_t(-1).value


def test_workspace_size():
    lib = abi.load()
    d = desc()
    assert lib.kda_prefill_workspace_size(ctypes.byref(d), 1, 64) == 0  # fp32 vector-ALU path needs none
    bad = desc(gate_lower_bound=math.nan)
    assert lib.kda_prefill_workspace_size(ctypes.byref(bad), 1, 64) == ctypes.c_size_t(-1).value


def test_timing_read_without_records_is_empty():
    # no GPU needed: with nothing recorded the read touches no event
    lib = abi.load()
    assert lib.kda_timing_read(None, None, 0) == 0
    assert abi.timing_enable(True) is False
    assert abi.timing_enable(False) is True
    assert abi.timing_read() == []


def test_noalloc_prefill_refuses_requests_beyond_its_scratch():
    # the fixed scratch holds 64 MiB per GPU: at H = 32, d = 128 (matrix-core path) 1472 tokens of one
    # sequence fit, 1473 do not; the refusal comes before any HIP call or pointer check
    lib = abi.load()
    d = desc(num_heads=32, head_dim_k=128, head_dim_v=128, chunk_size=64, io_dtype=abi.KDA_BF16)
    assert lib.kda_prefill_workspace_size(ctypes.byref(d), 1, 1472) <= (64 << 20)
    assert lib.kda_prefill_workspace_size(ctypes.byref(d), 1, 1473) > (64 << 20)

    def call(B, T, ptr=FAKE):
        return lib.kda_prefill_noalloc(ctypes.byref(d), B, T, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None)

    assert call(1, 1473) == abi.KDA_ERR_UNSUPPORTED
    msg = lib.kda_last_error()
    assert b"kda_prefill_noalloc" in msg and b"more than the library's fixed" in msg
    assert call(2, 705) == abi.KDA_ERR_UNSUPPORTED
    assert call(1, 1472, ptr=0) == abi.KDA_ERR_INVALID_ARGUMENT  # within the limit: pointers are checked next
    assert call(0, 5000, ptr=0) == abi.KDA_OK and call(1, 0, ptr=0) == abi.KDA_OK  # empty calls are no-ops
    assert lib.kda_prefill_noalloc(ctypes.byref(desc(gate_lower_bound=math.nan)), 1, 8, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, None) == abi.KDA_ERR_INVALID_ARGUMENT


def test_measure_stream_validation():
    lib = abi.load()
    P = ctypes.c_void_p
    assert lib.kda_measure_stream(None, None, 16, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"dst is null" in lib.kda_last_error()
    assert lib.kda_measure_stream(P(8), None, 16, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_measure_stream(P(16), P(24), 16, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"src is not 16-byte aligned" in lib.kda_last_error()
    assert lib.kda_measure_stream(P(16), P(32), 15, None) == abi.KDA_ERR_INVALID_ARGUMENT
    assert b"multiple of 16" in lib.kda_last_error()
