"""GPU parity: the HIP library, called through its C ABI, against the float64 oracle.

Small cases compare every element; full-size workloads run the library in the
exact launch configuration the benchmark times and compare the heads /
sequences the oracle computes one by one (heads are independent in this
layer), plus properties that hold at any size (chained == single-shot,
bit-identical reruns).
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_kda_amd import abi
from hybrid_linear_attention_kda_amd import inputs as I
from hybrid_linear_attention_kda_amd import tensors as TT
import parity_util as pu
from oracle import kda_oracle as O
from parity_util import TOL, TOL_BF16_OUT, head_channels, oracle_layer, oracle_prefilled, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dev_state(wl, inp, state=None, conv=None):
    s = inp["state0"] if state is None else state
    c = inp["conv_state0"] if conv is None else conv
    return (torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).to(DEV),
            TT.to_device(c, wl.io, DEV))


def _workspace(layer, B, T):
    n = abi.kda_prefill_workspace_size(layer, B, T)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=DEV) if n else None


def _gpu_prefill(wl, inp, layer, t0, t1, state, conv, out_dtype=torch.float32):
    tok = TT.token_tensors(wl, inp, t0, t1, DEV)
    out = torch.empty((wl.B, t1 - t0, wl.H * wl.dv), dtype=out_dtype, device=DEV)
    abi.kda_prefill(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], state, conv, out,
                    workspace=_workspace(layer, wl.B, t1 - t0))
    return out


def _check(name, got, ref, tol):
    e = rel_err(TT.to_host_f64(got) if isinstance(got, torch.Tensor) else got, ref)
    say(f"  {name}: rel err {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: {e:.3e} > {tol:.0e}"
    return e


# ---------------------------------------------------------------------------
# Tiny fp32 layer (every element)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [64, 1, 5, 45, 17])
def test_tiny_fp32_prefill(T):
    wl = I.WORKLOADS["tiny_fp32"].with_(T=T)
    say(f"case tiny_fp32 prefill T={T}")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, T, inp["state0"], inp["conv_state0"])
    tol = TOL["f32"]
    _check("out", out, ref["out"], tol)
    _check("state", st, ref["state"], tol)
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_tiny_fp32_split_prefill_5_plus_7():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=12)
    say("case tiny_fp32 split 5+7")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    o1 = _gpu_prefill(wl, inp, layer, 0, 5, st, cs)
    o2 = _gpu_prefill(wl, inp, layer, 5, 12, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 12, inp["state0"], inp["conv_state0"])
    _check("out", torch.cat([o1, o2], dim=1), ref["out"], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_tiny_fp32_nonzero_initial_state_and_conv_state():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=40, B=2)
    say("case tiny_fp32 nonzero initial state B=2 T=40")
    inp = I.generate(wl)
    rng = np.random.default_rng(5)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.5).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "f32")
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, 40, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 40, S0, C0)
    _check("out", out, ref["out"], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_tiny_fp32_decode_chain_equals_oracle():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=10, B=3)
    say("case tiny_fp32 decode chain B=3 T=10")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    outs = []
    for t in range(10):
        tok = TT.token_tensors(wl, inp, t, t + 1, DEV)
        out = torch.empty((3, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
        abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out)
        outs.append(out)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 10, inp["state0"], inp["conv_state0"])
    _check("out", torch.cat(outs, dim=1), ref["out"], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_tiny_fp32_verify_rollback_replay():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=8, B=4, prefix_T=6)
    say("case tiny_fp32 verify + rollback + replay")
    inp = I.generate(wl)
    pre = oracle_layer(wl, inp, 0, 6, inp["state0"], inp["conv_state0"])
    S0, C0 = pre["state"].astype(np.float32), pre["conv_state"].astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    tok = TT.token_tensors(wl, inp, 6, 14, DEV)
    snaps = torch.empty((4, 8, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out = torch.empty((4, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, snaps, out)
    torch.cuda.synchronize()
    ver = oracle_layer(wl, inp, 6, 14, S0, C0, record_states=True)
    _check("verify out", out, ver["out"], TOL["f32"])
    _check("snapshots", snaps, ver["states"], TOL["f32"])
    _check("live state untouched", st, S0, 0.0)
    accepted = [0, 3, 8, 5]
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st, cs)
    torch.cuda.synchronize()
    for b, m in enumerate(accepted):
        ref_s = S0[b] if m == 0 else ver["states"][b, m - 1]
        _check(f"rolled-back state b={b} m={m}", st[b], ref_s, TOL["f32"])
        sub = dict(inp)
        for k in ("qkv", "f", "beta", "g_out"):
            sub[k] = inp[k][b:b + 1]
        ref_c = oracle_layer(wl, sub, 6, 6 + m, S0[b:b + 1], C0[b:b + 1])["conv_state"][0]
        _check(f"rolled-back conv b={b} m={m}", cs[b], ref_c, 0.0)


def _bit_equal(name, a, b):
    same = torch.equal(a, b)
    say(f"  {name}: bit-identical {same}")
    assert same, name


def test_tiny_fp32_verify_tape_and_commit():
    wl = I.WORKLOADS["tiny_fp32"].with_(T=8, B=4, prefix_T=6)
    say("case tiny_fp32 verify with replay tape + commit")
    inp = I.generate(wl)
    pre = oracle_layer(wl, inp, 0, 6, inp["state0"], inp["conv_state0"])
    S0, C0 = pre["state"].astype(np.float32), pre["conv_state"].astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV)
    tok = TT.token_tensors(wl, inp, 6, 14, DEV)
    # snapshot path
    st1, cs1 = _dev_state(wl, inp, S0, C0)
    snaps = torch.empty((4, 8, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out1 = torch.empty((4, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st1, cs1, snaps, out1)
    # tape path
    st2, cs2 = _dev_state(wl, inp, S0, C0)
    assert abi.kda_verify_tape_size(layer, 4, 8) == 4 * 8 * wl.H * 3 * wl.dk * 4
    tape = torch.empty((4, 8, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out2 = torch.empty_like(out1)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st2, cs2, tape, out2)
    torch.cuda.synchronize()
    _bit_equal("verify out, tape vs snapshot path", out2, out1)
    _check("live state untouched", st2, S0, 0.0)
    sub = I.split_tokens(inp, 6, 14)
    ref = O.kda_verify_tape(pu.params(wl, inp), sub["qkv"], sub["f"], sub["beta"], sub["g_out"], S0, C0)
    _check("verify out", out2, ref["out"], TOL["f32"])
    for j, name in enumerate(("alpha", "k", "u")):
        _check(f"tape {name}", tape[:, :, :, j], ref["tape"][:, :, :, j], TOL["f32"])
    accepted = [0, 3, 8, 5]
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st1, cs1)
    abi.kda_commit_tape(layer, accepted, tape, tok["qkv"], st2, cs2)
    torch.cuda.synchronize()
    _bit_equal("committed state, tape vs snapshot path", st2, st1)
    _bit_equal("committed conv state, tape vs snapshot path", cs2, cs1)
    ref_s, ref_c = O.kda_commit_tape(pu.params(wl, inp), accepted, ref["tape"], sub["qkv"], S0, C0)
    _check("committed state", st2, ref_s, TOL["f32"])
    _check("committed conv state", cs2, ref_c, 0.0)


def test_tiny_fp32_verify_max_draft_length():
    # the longest draft block the boundary takes (T_d = 255): 31 full groups of the verify kernel's
    # 8-token input prefetch and a partial one, and the tape commit's 8-token staging with a partial
    # last group; snapshots, rollback, tape and commit against the oracle
    Td = 255
    wl = I.WORKLOADS["tiny_fp32"].with_(T=Td, B=3, prefix_T=6, seed=77)
    say(f"case tiny_fp32 verify T_d={Td} (the maximum) + rollback, tape + commit")
    inp = I.generate(wl)
    pre = oracle_layer(wl, inp, 0, 6, inp["state0"], inp["conv_state0"])
    S0, C0 = pre["state"].astype(np.float32), pre["conv_state"].astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV)
    tok = TT.token_tensors(wl, inp, 6, 6 + Td, DEV)
    st1, cs1 = _dev_state(wl, inp, S0, C0)
    snaps = torch.empty((3, Td, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out1 = torch.empty((3, Td, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st1, cs1, snaps, out1)
    st2, cs2 = _dev_state(wl, inp, S0, C0)
    tape = torch.empty((3, Td, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out2 = torch.empty_like(out1)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st2, cs2, tape, out2)
    torch.cuda.synchronize()
    ver = oracle_layer(wl, inp, 6, 6 + Td, S0, C0, record_states=True)
    _check("verify out", out1, ver["out"], TOL["f32"])
    _check("snapshots", snaps, ver["states"], TOL["f32"])
    _bit_equal("verify out, tape vs snapshot path", out2, out1)
    accepted = [0, Td, 131]
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st1, cs1)
    abi.kda_commit_tape(layer, accepted, tape, tok["qkv"], st2, cs2)
    torch.cuda.synchronize()
    _bit_equal("committed state, tape vs snapshot path", st2, st1)
    _bit_equal("committed conv state, tape vs snapshot path", cs2, cs1)
    for b, m in enumerate(accepted):
        ref_s = S0[b] if m == 0 else ver["states"][b, m - 1]
        _check(f"state b={b} m={m}", st1[b], ref_s, TOL["f32"])
        sub = dict(inp)
        for k in ("qkv", "f", "beta", "g_out"):
            sub[k] = inp[k][b:b + 1]
        ref_c = oracle_layer(wl, sub, 6, 6 + m, S0[b:b + 1], C0[b:b + 1])["conv_state"][0]
        _check(f"conv state b={b} m={m}", cs1[b], ref_c, 0.0)


def test_verify_tape_b16_full_size_with_commit():
    wl = I.WORKLOADS["verify_b16"]
    say("case verify_b16 full size (B=16, T_d=8, H=32, d=128) with replay tape + commit, 16 distinct states")
    inp = I.generate(wl)
    S0, C0 = oracle_prefilled(wl, inp, n_pre=16)
    layer = TT.make_layer(wl, inp, DEV)
    t0 = wl.prefix_T
    tok = TT.token_tensors(wl, inp, t0, t0 + wl.T, DEV)
    st1, cs1 = _dev_state(wl, inp, S0, C0)
    snaps = torch.empty((wl.B, wl.T, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out1 = torch.empty((wl.B, wl.T, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st1, cs1, snaps, out1)
    st2, cs2 = _dev_state(wl, inp, S0, C0)
    tape = torch.empty((wl.B, wl.T, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out2 = torch.empty_like(out1)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st2, cs2, tape, out2)
    torch.cuda.synchronize()
    _bit_equal("verify out, tape vs snapshot path", out2, out1)
    accepted = [int(m) for m in inp["accepted"]]
    say(f"  accepted = {accepted}")
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st1, cs1)
    abi.kda_commit_tape(layer, accepted, tape, tok["qkv"], st2, cs2)
    torch.cuda.synchronize()
    _bit_equal("committed state, tape vs snapshot path", st2, st1)
    _bit_equal("committed conv state, tape vs snapshot path", cs2, cs1)
    sub = I.split_tokens(inp, t0, t0 + wl.T)
    ref = O.kda_verify_tape(pu.params(wl, inp), sub["qkv"], sub["f"], sub["beta"], sub["g_out"], S0, C0)
    _check("verify out", out2, ref["out"], TOL["bf16"])
    ref_s, ref_c = O.kda_commit_tape(pu.params(wl, inp), accepted, ref["tape"], sub["qkv"], S0, C0)
    _check("committed state", st2, ref_s, TOL["bf16"])
    _check("committed conv state", cs2, ref_c, 0.0)


# ---------------------------------------------------------------------------
# bf16 layers at the model's head size (every element)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [200, 64, 1])
def test_bf16_prefill_four_heads(T):
    wl = I.WORKLOADS["prefill_t4096"].with_(T=T, H=4, B=2, seed=11)
    say(f"case bf16 prefill H=4 B=2 T={T}")
    inp = I.generate(wl)
    rng = np.random.default_rng(T)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, T, S0, C0)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)
    # bf16 output mode: one extra rounding of each output element
    layer16 = TT.make_layer(wl, inp, DEV, out="bf16")
    st2, cs2 = _dev_state(wl, inp, S0, C0)
    out16 = _gpu_prefill(wl, inp, layer16, 0, T, st2, cs2, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _check("out (bf16 output)", out16, ref["out"], TOL_BF16_OUT)


@pytest.mark.parametrize("W,lb", [(1, -5.0), (2, -5.0), (3, -5.0), (4, -0.25), (4, -5.5), (4, 0.0), (4, -0.1),
                                  (4, -5.6), (4, -8.0), (4, -30.0)])
def test_bf16_prefill_conv_widths_and_gate_bounds(W, lb):
    # the matrix-core path takes conv widths 1..4 and every bound <= 0: start-anchored sub-chunks for
    # -5.5 <= lb <= 0 (lb = 0: no decay at all), end-anchored ones with exact diagonal blocks below it
    wl = I.WORKLOADS["prefill_t4096"].with_(T=150, H=2, B=2, W=W, lb=lb, seed=30 + W)
    say(f"case bf16 prefill W={W} lb={lb} H=2 B=2 T=150")
    inp = I.generate(wl)
    rng = np.random.default_rng(W)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
    layer = TT.make_layer(wl, inp, DEV)
    assert abi.kda_prefill_workspace_size(layer, 2, 150) > 0, "the matrix-core path"
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, 150, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 150, S0, C0)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    if W > 1:
        _check("conv_state", cs, ref["conv_state"], 0.0)


@pytest.mark.parametrize("W", [1, 8])
def test_tiny_fp32_conv_width_extremes_prefill_decode_tape(W):
    # conv widths 1 (no conv state) and 8 (the widest supported): fp32 prefill of a prefix, then a
    # decode step, then a tape verify of 8 tokens and its commit
    wl = I.WORKLOADS["tiny_fp32"].with_(T=8, B=2, W=W, prefix_T=6, seed=40 + W)
    say(f"case tiny_fp32 W={W}: prefill 5, decode 1, tape verify 8 + commit")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, 5, st, cs)
    tok = TT.token_tensors(wl, inp, 5, 6, DEV)
    out1 = torch.empty((2, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 6, inp["state0"], inp["conv_state0"])
    _check("prefill out", out, ref["out"][:, :5], TOL["f32"])
    _check("decode out", out1, ref["out"][:, 5:6], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    if W > 1:
        _check("conv_state", cs, ref["conv_state"], 0.0)
    S6, C6 = ref["state"].astype(np.float32), ref["conv_state"].astype(np.float32)
    tok = TT.token_tensors(wl, inp, 6, 14, DEV)
    tape = torch.empty((2, 8, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out8 = torch.empty((2, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, tape, out8)
    accepted = [3, 8]
    abi.kda_commit_tape(layer, accepted, tape, tok["qkv"], st, cs)
    torch.cuda.synchronize()
    sub = I.split_tokens(inp, 6, 14)
    rv = O.kda_verify_tape(pu.params(wl, inp), sub["qkv"], sub["f"], sub["beta"], sub["g_out"], S6, C6)
    _check("tape verify out", out8, rv["out"], TOL["f32"])
    ref_s, ref_c = O.kda_commit_tape(pu.params(wl, inp), accepted, rv["tape"], sub["qkv"], S6, C6)
    _check("committed state", st, ref_s, TOL["f32"])
    if W > 1:
        _check("committed conv state", cs, ref_c, 0.0)


# ---------------------------------------------------------------------------
# The softplus decay branch (no lower bound)
# ---------------------------------------------------------------------------

def test_softplus_tiny_fp32_prefill_decode_verify_rollback_tape():
    # fp32 io: prefill 5 tokens, one decode step, then an 8-token draft block through the snapshot
    # verify + rollback and through the tape verify + commit, all with the softplus gate
    wl = I.WORKLOADS["tiny_fp32"].with_(T=8, B=4, prefix_T=6, gate="softplus", seed=50)
    say("case tiny_fp32 softplus: prefill 5, decode 1, verify 8 + rollback, tape verify 8 + commit")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    assert layer.gate_kind == abi.KDA_GATE_SOFTPLUS and np.isnan(layer.lb)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, 5, st, cs)
    tok = TT.token_tensors(wl, inp, 5, 6, DEV)
    out1 = torch.empty((4, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 6, inp["state0"], inp["conv_state0"])
    _check("prefill out", out, ref["out"][:, :5], TOL["f32"])
    _check("decode out", out1, ref["out"][:, 5:6], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)
    S6, C6 = ref["state"].astype(np.float32), ref["conv_state"].astype(np.float32)
    tok = TT.token_tensors(wl, inp, 6, 14, DEV)
    snaps = torch.empty((4, 8, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out8 = torch.empty((4, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    st2, cs2 = _dev_state(wl, inp, S6, C6)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st2, cs2, snaps, out8)
    accepted = [0, 3, 8, 5]
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st2, cs2)
    torch.cuda.synchronize()
    ver = oracle_layer(wl, inp, 6, 14, S6, C6, record_states=True)
    _check("verify out", out8, ver["out"], TOL["f32"])
    _check("snapshots", snaps, ver["states"], TOL["f32"])
    for b, m in enumerate(accepted):
        _check(f"rolled-back state b={b} m={m}", st2[b], S6[b] if m == 0 else ver["states"][b, m - 1], TOL["f32"])
    st3, cs3 = _dev_state(wl, inp, S6, C6)
    tape = torch.empty((4, 8, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out8t = torch.empty_like(out8)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st3, cs3, tape, out8t)
    abi.kda_commit_tape(layer, accepted, tape, tok["qkv"], st3, cs3)
    torch.cuda.synchronize()
    _bit_equal("tape verify out == snapshot verify out", out8t, out8)
    _bit_equal("committed state == rolled-back state", st3, st2)
    _bit_equal("committed conv state == rolled-back conv state", cs3, cs2)


def test_softplus_bf16_prefill_then_decode():
    # bf16 io at the model's head size: the softplus branch on the matrix-core prefill (end-anchored
    # key columns, exact diagonal sub-chunk blocks), then a decode step continues each sequence
    wl = I.WORKLOADS["prefill_t4096"].with_(T=151, H=2, B=2, gate="softplus", prefix_T=0, seed=51)
    say("case bf16 softplus prefill 150 + decode 1 (H=2 B=2 d=128)")
    inp = I.generate(wl)
    rng = np.random.default_rng(51)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, 150, st, cs)
    tok = TT.token_tensors(wl, inp, 150, 151, DEV)
    out1 = torch.empty((2, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 151, S0, C0)
    _check("prefill out", out, ref["out"][:, :150], TOL["bf16"])
    _check("decode out", out1, ref["out"][:, 150:], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


@pytest.mark.parametrize("W", [1, 3])
def test_softplus_bf16_prefill_conv_widths_chained(W):
    # the softplus instance of the matrix-core prefill at conv widths 1 and 3, as two chained calls
    # (100 + 50 tokens) against one call and the oracle
    wl = I.WORKLOADS["prefill_t4096"].with_(T=150, H=2, B=2, W=W, gate="softplus", seed=54 + W)
    say(f"case bf16 softplus prefill W={W}, 100 + 50 chained vs single-shot")
    inp = I.generate(wl)
    rng = np.random.default_rng(60 + W)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    o1 = _gpu_prefill(wl, inp, layer, 0, 100, st, cs)
    o2 = _gpu_prefill(wl, inp, layer, 100, 150, st, cs)
    st1, cs1 = _dev_state(wl, inp, S0, C0)
    o = _gpu_prefill(wl, inp, layer, 0, 150, st1, cs1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 150, S0, C0)
    _check("chained out", torch.cat([o1, o2], dim=1), ref["out"], TOL["bf16"])
    _check("single-shot out", o, ref["out"], TOL["bf16"])
    _check("chained state", st, ref["state"], TOL["bf16"])
    _check("single-shot state", st1, ref["state"], TOL["bf16"])
    if W > 1:
        _check("conv_state", cs, ref["conv_state"], 0.0)
        assert torch.equal(cs, cs1)


@pytest.mark.parametrize("shift", [-12.0, 8.0, 60.0])
def test_softplus_bf16_prefill_extreme_decays(shift):
    # f + dt_bias shifted so the decay is nearly absent (-12: g ~ -A e^-12), strong (8: g ~ -8 A)
    # or far past any sub-chunk bound (60: g ~ -60 A, floored at -100), with every fourth token
    # unshifted so strong and weak decays mix inside the sub-chunks; T = 150 (a partial chunk)
    wl = I.WORKLOADS["prefill_t4096"].with_(T=150, H=2, B=1, gate="softplus", seed=52)
    say(f"case bf16 softplus prefill, f shifted by {shift} on three tokens of four")
    inp = dict(I.generate(wl))
    f = inp["f"].astype(np.float64)
    f[:, np.arange(150) % 4 != 0] += shift
    inp["f"] = I.round_to_io(f, "bf16")
    rng = np.random.default_rng(53)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0)
    out = _gpu_prefill(wl, inp, layer, 0, 150, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 150, S0, inp["conv_state0"])
    assert torch.isfinite(out).all()
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])


# ---------------------------------------------------------------------------
# Variable-length prefill over a state pool (every element)
# ---------------------------------------------------------------------------

def _varlen_case(wl, lens, slots, num_slots, seed, out_dtype=torch.float32):
    """Run kda_prefill_varlen on a packed batch and the oracle per sequence; returns both."""
    total = sum(lens)
    cu = I.cu_seqlens(lens)
    inp = I.generate(wl.with_(B=1, T=total))
    rng = np.random.default_rng(seed)
    pool = (rng.standard_normal((num_slots, wl.H, wl.dk, wl.dv)) * 0.3).astype(np.float32)
    cpool = I.round_to_io(rng.standard_normal((num_slots, wl.c_qkv, wl.W - 1)), wl.io)
    layer = TT.make_layer(wl, inp, DEV, out="bf16" if out_dtype == torch.bfloat16 else "f32")
    st = torch.from_numpy(pool).to(DEV)
    cs = TT.to_device(cpool, wl.io, DEV)
    tok = {k: v[0] for k, v in TT.token_tensors(wl, inp, 0, total, DEV).items()}
    out = torch.empty((total, wl.H * wl.dv), dtype=out_dtype, device=DEV)
    n = abi.kda_prefill_varlen_workspace_size(layer, cu)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=DEV) if n else None
    abi.kda_prefill_varlen(layer, cu, slots, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out,
                           workspace=ws)
    torch.cuda.synchronize()
    pk = {k: inp[k][0] for k in ("qkv", "f", "beta", "g_out")}
    ref = O.kda_prefill_varlen(pu.params(wl, inp), cu, slots, pk["qkv"], pk["f"], pk["beta"], pk["g_out"],
                               pool, cpool)
    return out, st, cs, ref, pool, cpool


def test_bf16_varlen_prefill_mixed_lengths_and_slots():
    # ragged lengths (empty, one token, exactly one chunk, partial chunks, several chunks), a slot
    # permutation and a pool slot no sequence names
    wl = I.WORKLOADS["prefill_t4096"].with_(H=4, seed=21)
    lens = [0, 1, 64, 100, 257, 3]
    slots = [2, 5, 0, 3, 1, 4]
    say(f"case bf16 varlen H=4 lengths {lens} slots {slots} (pool of 7)")
    out, st, cs, ref, pool, cpool = _varlen_case(wl, lens, slots, 7, seed=5)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state pool", st, ref["state"], TOL["bf16"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)
    _check("unnamed slot and empty sequence's slot untouched", st[[6, 2]], pool[[6, 2]], 0.0)


def test_bf16_varlen_equals_batched_prefill():
    # equal lengths: the packed call is bit-identical to kda_prefill on B sequences
    wl = I.WORKLOADS["prefill_t4096"].with_(H=4, B=3, T=150, seed=22)
    say("case bf16 varlen 3 x 150 tokens vs batched prefill")
    inp = I.generate(wl)
    rng = np.random.default_rng(9)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
    layer = TT.make_layer(wl, inp, DEV)
    st1, cs1 = _dev_state(wl, inp, S0, C0)
    out1 = _gpu_prefill(wl, inp, layer, 0, 150, st1, cs1)
    st2, cs2 = _dev_state(wl, inp, S0, C0)
    tok = TT.token_tensors(wl, inp, 0, 150, DEV)
    out2 = torch.empty((450, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    cu = [0, 150, 300, 450]
    ws = torch.empty(abi.kda_prefill_varlen_workspace_size(layer, cu), dtype=torch.uint8, device=DEV)
    abi.kda_prefill_varlen(layer, cu, None, tok["qkv"].reshape(450, -1), tok["f"].reshape(450, -1),
                           tok["beta"].reshape(450, -1), tok["g_out"].reshape(450, -1), st2, cs2, out2, workspace=ws)
    torch.cuda.synchronize()
    _bit_equal("out", out2, out1.reshape(450, -1))
    _bit_equal("state", st2, st1)
    _bit_equal("conv state", cs2, cs1)


def test_bf16_varlen_more_sequences_than_one_launch_holds():
    # 150 short sequences (over the 128 of one launch's table), two heads
    wl = I.WORKLOADS["prefill_t4096"].with_(H=2, seed=23)
    rng = np.random.default_rng(3)
    lens = [int(x) for x in rng.integers(0, 6, size=150)]
    slots = [int(x) for x in rng.permutation(160)[:150]]
    say(f"case bf16 varlen 150 sequences, {sum(lens)} tokens, pool of 160")
    out, st, cs, ref, pool, cpool = _varlen_case(wl, lens, slots, 160, seed=6)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state pool", st, ref["state"], TOL["bf16"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)


def test_bf16_varlen_prefill_softplus():
    wl = I.WORKLOADS["prefill_t4096"].with_(H=2, seed=24, gate="softplus")
    lens = [0, 1, 70, 130]
    say(f"case bf16 varlen softplus H=2 lengths {lens}")
    out, st, cs, ref, pool, cpool = _varlen_case(wl, lens, [1, 3, 0, 2], 4, seed=8)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state pool", st, ref["state"], TOL["bf16"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)


@pytest.mark.parametrize("out_kind", ["bf16", "f32"])
def test_varlen_full_size_bench_packing_all_heads(out_kind):
    # the packed call the benchmark times: the 4096 tokens of prefill_t4096 as 16 sequences of the
    # seeded length mix, all 32 heads, one slot per sequence; the oracle runs every sequence on every
    # head; bf16 output at the one-rounding bound, fp32 output at the 2e-3 bar
    wl = I.WORKLOADS["prefill_t4096"]
    lens = I.varlen_lengths(wl.T, 16, 8)
    total = sum(lens)
    cu = I.cu_seqlens(lens)
    say(f"case varlen full size: H=32, 16 sequences {lens}, {out_kind} out, oracle on every head")
    inp = I.generate(wl.with_(B=1, T=total))
    rng = np.random.default_rng(11)
    pool = (rng.standard_normal((16, wl.H, wl.dk, wl.dv)) * 0.3).astype(np.float32)
    cpool = I.round_to_io(rng.standard_normal((16, wl.c_qkv, wl.W - 1)), wl.io)
    layer = TT.make_layer(wl, inp, DEV, out=out_kind)
    st = torch.from_numpy(pool).to(DEV)
    cs = TT.to_device(cpool, wl.io, DEV)
    tok = {k: v[0] for k, v in TT.token_tensors(wl, inp, 0, total, DEV).items()}
    odt = torch.bfloat16 if out_kind == "bf16" else torch.float32
    out = torch.empty((total, wl.H * wl.dv), dtype=odt, device=DEV)
    ws = torch.empty(abi.kda_prefill_varlen_workspace_size(layer, cu), dtype=torch.uint8, device=DEV)
    abi.kda_prefill_varlen(layer, cu, None, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out,
                           workspace=ws)
    torch.cuda.synchronize()
    pk = {k: inp[k][0] for k in ("qkv", "f", "beta", "g_out")}
    ref = O.kda_prefill_varlen(pu.params(wl.with_(T=total), inp), cu, None, pk["qkv"], pk["f"], pk["beta"],
                               pk["g_out"], pool, cpool)
    _check("out", out, ref["out"], TOL_BF16_OUT if out_kind == "bf16" else TOL["bf16"])
    _check("state pool", st, ref["state"], TOL["bf16"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)


def test_tiny_fp32_varlen_prefill():
    wl = I.WORKLOADS["tiny_fp32"]
    lens = [5, 0, 17, 64, 1]
    say(f"case fp32 varlen H=2 d=16 lengths {lens}")
    out, st, cs, ref, pool, cpool = _varlen_case(wl, lens, [4, 0, 1, 3, 2], 6, seed=7)
    _check("out", out, ref["out"], TOL["f32"])
    _check("state pool", st, ref["state"], TOL["f32"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)


@pytest.mark.parametrize("T,gate", [(100, "sigmoid"), (33, "sigmoid"), (100, "softplus")])
def test_fp32_prefill_head_size_128(T, gate):
    # fp32 io at d = 128 runs the vector-ALU chunked prefill (internal chunk 32)
    wl = I.WORKLOADS["prefill_t4096"].with_(T=T, H=2, B=2, io="f32", seed=12, gate=gate)
    say(f"case fp32 prefill d=128 H=2 B=2 T={T} gate {gate}")
    inp = I.generate(wl)
    rng = np.random.default_rng(100 + T)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = rng.standard_normal(inp["conv_state0"].shape).astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, T, S0, C0)
    _check("out", out, ref["out"], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_fp32_prefill_head_size_128_bf16_out():
    # bf16 out keeps one workgroup per (sequence, head), the RMSNorm fused into the prefill kernel
    # (fp32 out with few pairs splits the value columns over workgroups and norms in a second pass)
    wl = I.WORKLOADS["prefill_t4096"].with_(T=70, H=2, B=2, io="f32", seed=13)
    say("case fp32 io, bf16 out, d=128 H=2 B=2 T=70")
    inp = I.generate(wl)
    rng = np.random.default_rng(170)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = rng.standard_normal(inp["conv_state0"].shape).astype(np.float32)
    layer = TT.make_layer(wl, inp, DEV, out="bf16")
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, 70, st, cs, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 70, S0, C0)
    _check("out", out, ref["out"], TOL_BF16_OUT)
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


@pytest.mark.parametrize("d,io", [(32, "f32"), (64, "f32"), (64, "bf16")])
def test_vector_alu_prefill_head_sizes_32_64(d, io):
    # head sizes the matrix-core path does not take: internal chunk 64, the value columns split over
    # two (d = 32) or four (d = 64, 16 columns each) workgroups per head, one full chunk and a ragged
    # tail; the arithmetic is fp32 throughout for bf16 io too
    wl = I.WORKLOADS["prefill_t4096"].with_(T=100, H=2, B=2, dk=d, dv=d, io=io, seed=14)
    say(f"case vector-ALU prefill d={d} io={io} H=2 B=2 T=100")
    inp = I.generate(wl)
    rng = np.random.default_rng(200 + d)
    S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
    C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), io)
    layer = TT.make_layer(wl, inp, DEV, out="f32")
    st, cs = _dev_state(wl, inp, S0, C0)
    out = _gpu_prefill(wl, inp, layer, 0, 100, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 100, S0, C0)
    _check("out", out, ref["out"], TOL["f32"])
    _check("state", st, ref["state"], TOL["f32"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_fp32_varlen_prefill_head_size_128():
    # split value columns with the state and conv-state pools updated in place, ragged lengths
    wl = I.WORKLOADS["prefill_t4096"].with_(H=2, io="f32", seed=23)
    lens = [0, 1, 33, 70]
    slots = [1, 3, 0, 2]
    say(f"case fp32 varlen d=128 H=2 lengths {lens} slots {slots} (pool of 5)")
    out, st, cs, ref, pool, cpool = _varlen_case(wl, lens, slots, 5, seed=9)
    _check("out", out, ref["out"], TOL["f32"])
    _check("state pool", st, ref["state"], TOL["f32"])
    _check("conv-state pool", cs, ref["conv_state"], 0.0)
    _check("unnamed slot and empty sequence's slot untouched", st[[4, 1]], pool[[4, 1]], 0.0)


# ---------------------------------------------------------------------------
# Edge cases: the L2 clamp, weak decay over long sequences, a visible query scale
# ---------------------------------------------------------------------------

def _tiny_qk_heads(wl, inp, t0=0):
    # raw q and k of head 0, and raw q of head 1, scaled to ~1e-8: after the conv and SiLU their
    # norms are ~1e-7, below the 1e-6 clamp, so x / max(||x||, eps) divides by eps itself
    inp = dict(inp)
    qkv = inp["qkv"].astype(np.float64).copy()
    H, d = wl.H, wl.dk
    for ch in (np.arange(0, d), np.arange(H * d, H * d + d), np.arange(d, 2 * d)):
        qkv[:, t0:, ch] *= 1e-8
    inp["qkv"] = I.round_to_io(qkv, wl.io)
    return inp


def test_l2_clamp_prefill_and_decode():
    # bf16 at d = 128: the matrix-core prefill of 130 tokens, then a decode step and a tape verify of
    # 8 tokens, with heads whose q / k norms sit below the clamp on every token
    wl = I.WORKLOADS["prefill_t4096"].with_(T=139, H=4, B=2, seed=70)
    say("case L2 clamp: heads 0 (q and k) and 1 (q) below eps; prefill 130, decode 1, tape verify 8")
    inp = _tiny_qk_heads(wl, I.generate(wl))
    p = pu.params(wl, inp)
    q, k, _, _, _ = O.prologue(p, inp["qkv"][0, :130], inp["f"][0, :130], inp["conv_state0"][0])
    qn = np.sqrt(np.sum((q / p.scale) ** 2, axis=-1))  # normalised length, < 1 where clamped
    assert np.all(qn[:, 0] < 0.5) and np.all(qn[:, 1] < 0.5) and np.all(np.abs(qn[:, 2:] - 1) < 1e-9)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, 130, st, cs)
    tok = TT.token_tensors(wl, inp, 130, 131, DEV)
    out1 = torch.empty((2, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 131, inp["state0"], inp["conv_state0"])
    assert torch.isfinite(out).all() and torch.isfinite(out1).all()
    _check("prefill out", out, ref["out"][:, :130], TOL["bf16"])
    _check("decode out", out1, ref["out"][:, 130:], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)
    S1, C1 = ref["state"].astype(np.float32), ref["conv_state"].astype(np.float32)
    tok = TT.token_tensors(wl, inp, 131, 139, DEV)
    tape = torch.empty((2, 8, wl.H, 3, wl.dk), dtype=torch.float32, device=DEV)
    out8 = torch.empty((2, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block_tape(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, tape, out8)
    torch.cuda.synchronize()
    sub = I.split_tokens(inp, 131, 139)
    rv = O.kda_verify_tape(p, sub["qkv"], sub["f"], sub["beta"], sub["g_out"], S1, C1)
    _check("tape verify out", out8, rv["out"], TOL["bf16"])
    _check("tape k rows (clamped heads included)", tape[:, :, :, 1], rv["tape"][:, :, :, 1], TOL["bf16"])


@pytest.mark.parametrize("gate", ["sigmoid", "softplus"])
def test_weak_decay_t4096(gate):
    # consistently weak decay for a whole 4096-token sequence on the matrix-core prefill: the bounded
    # gate with dt_bias shifted by -4 on half of every head's channels (sigmoid(A (f - 4)) ~ 0.02, so
    # g ~ -0.1 there), and the softplus branch with f shifted by -12 on every token (g ~ -A e^-12)
    wl = I.WORKLOADS["prefill_t4096"].with_(H=8, gate=gate, seed=71)
    inp = dict(I.generate(wl))
    if gate == "sigmoid":
        dtb = inp["dt_bias"].copy()
        dtb.reshape(wl.H, wl.dk)[:, ::2] -= 4.0
        inp["dt_bias"] = dtb
        say("case weak decay, bounded gate: dt_bias - 4 on half the channels, T=4096, H=8")
    else:
        inp["f"] = I.round_to_io(inp["f"].astype(np.float64) - 12.0, "bf16")
        say("case weak decay, softplus branch: f - 12 on every token, T=4096, H=8")
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, wl.T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, wl.T, inp["state0"], inp["conv_state0"])
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])


@pytest.mark.parametrize("lb", [-8.0, -0.1, 0.0])
def test_gate_bound_outside_the_start_anchored_range_t4096(lb):
    # 4096 tokens on the matrix-core path at a bound below the start-anchored range (-8: end-anchored
    # sub-chunks with exact diagonal blocks) and at a weak bound (-0.1: the state keeps most of its
    # past, which split W carries within the tolerance)
    wl = I.WORKLOADS["prefill_t4096"].with_(H=8, lb=lb, seed=73)
    say(f"case bounded gate lb={lb}, T=4096, H=8, matrix-core prefill")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    assert abi.kda_prefill_workspace_size(layer, 1, wl.T) > 0, "the matrix-core path"
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, wl.T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, wl.T, inp["state0"], inp["conv_state0"])
    assert torch.isfinite(out).all()
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_query_scale_visible_through_the_norm():
    # rms_eps = 1 and scale = 0.05 keep the RMSNorm from cancelling the query scale: out depends on
    # where (and whether) the scale is applied; matrix-core prefill, decode step and snapshot verify
    wl = I.WORKLOADS["prefill_t4096"].with_(T=209, H=4, B=2, seed=72)
    say("case query scale visible: rms_eps 1.0, scale 0.05; prefill 200, decode 1, verify 8")
    inp = dict(I.generate(wl))
    inp["rms_eps"] = 1.0
    inp["scale"] = 0.05
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, 200, st, cs)
    tok = TT.token_tensors(wl, inp, 200, 201, DEV)
    out1 = torch.empty((2, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out1)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, 201, inp["state0"], inp["conv_state0"])
    # the same layer at scale 1 differs by far more than the tolerance (the scale is visible)
    inp1 = dict(inp, scale=1.0)
    ref1 = oracle_layer(wl, inp1, 0, 201, inp["state0"], inp["conv_state0"])
    assert rel_err(ref1["out"], ref["out"]) > 0.5
    _check("prefill out", out, ref["out"][:, :200], TOL["bf16"])
    _check("decode out", out1, ref["out"][:, 200:], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    S1, C1 = ref["state"].astype(np.float32), ref["conv_state"].astype(np.float32)
    tok = TT.token_tensors(wl, inp, 201, 209, DEV)
    snaps = torch.empty((2, 8, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out8 = torch.empty((2, 8, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, snaps, out8)
    torch.cuda.synchronize()
    ver = oracle_layer(wl, inp, 201, 209, S1, C1, record_states=True)
    _check("verify out", out8, ver["out"], TOL["bf16"])
    _check("snapshots", snaps, ver["states"], TOL["bf16"])


# ---------------------------------------------------------------------------
# Full-size workloads, in the benchmark's launch configuration
# ---------------------------------------------------------------------------

def test_decode_b64_full_size():
    wl = I.WORKLOADS["decode_b64"]
    say("case decode_b64 full size (B=64, H=32, d=128), 16 distinct oracle pre-filled states")
    inp = I.generate(wl)
    S0, C0 = oracle_prefilled(wl, inp, n_pre=16)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    t0 = wl.prefix_T
    tok = TT.token_tensors(wl, inp, t0, t0 + 1, DEV)
    out = torch.empty((wl.B, 1, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_decode_step(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, t0, t0 + 1, S0, C0)
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)


def test_verify_b16_full_size_with_rollback():
    wl = I.WORKLOADS["verify_b16"]
    say("case verify_b16 full size (B=16, T_d=8, H=32, d=128) + rollback, 16 distinct pre-filled states")
    inp = I.generate(wl)
    S0, C0 = oracle_prefilled(wl, inp, n_pre=16)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp, S0, C0)
    t0 = wl.prefix_T
    tok = TT.token_tensors(wl, inp, t0, t0 + wl.T, DEV)
    snaps = torch.empty((wl.B, wl.T, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=DEV)
    out = torch.empty((wl.B, wl.T, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    abi.kda_verify_block(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, snaps, out)
    torch.cuda.synchronize()
    ver = oracle_layer(wl, inp, t0, t0 + wl.T, S0, C0, record_states=True)
    _check("verify out", out, ver["out"], TOL["bf16"])
    _check("snapshots", snaps, ver["states"], TOL["bf16"])
    accepted = [int(m) for m in inp["accepted"]]
    say(f"  accepted = {accepted}")
    abi.kda_rollback(layer, accepted, snaps, tok["qkv"], st, cs)
    torch.cuda.synchronize()
    ref_s = np.stack([S0[b] if m == 0 else ver["states"][b, m - 1] for b, m in enumerate(accepted)])
    _check("rolled-back state", st, ref_s, TOL["bf16"])
    ref_c = []
    for b, m in enumerate(accepted):
        sub = {k: inp[k][b:b + 1] for k in ("qkv", "f", "beta", "g_out")}
        sub.update({k: inp[k] for k in inp if k not in sub})
        ref_c.append(oracle_layer(wl, sub, t0, t0 + m, S0[b:b + 1], C0[b:b + 1])["conv_state"][0])
    _check("rolled-back conv", cs, np.stack(ref_c), 0.0)


@pytest.mark.parametrize("gate", ["sigmoid", "softplus"])
def test_prefill_t4096_full_size_all_heads(gate):
    wl = I.WORKLOADS["prefill_t4096"].with_(gate=gate)
    say(f"case prefill_t4096 full size (B=1, T=4096, H=32, d=128), gate {gate}, oracle on every head")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    out = _gpu_prefill(wl, inp, layer, 0, wl.T, st, cs)
    torch.cuda.synchronize()
    ref = oracle_layer(wl, inp, 0, wl.T, inp["state0"], inp["conv_state0"])
    _check("out", out, ref["out"], TOL["bf16"])
    _check("state", st, ref["state"], TOL["bf16"])
    _check("conv_state", cs, ref["conv_state"], 0.0)
    # per head too, so that one head's error is not hidden by another's larger values
    o64, s64 = TT.to_host_f64(out), TT.to_host_f64(st)
    worst = max(max(rel_err(o64[..., h * 128:(h + 1) * 128], ref["out"][..., h * 128:(h + 1) * 128]),
                    rel_err(s64[:, h], ref["state"][:, h])) for h in range(wl.H))
    say(f"  worst head: rel err {worst:.3e}")
    assert worst <= TOL["bf16"]
    # a second run on the same inputs is bit-identical (no atomics, fixed reduction order)
    st2, cs2 = _dev_state(wl, inp)
    out2 = _gpu_prefill(wl, inp, layer, 0, wl.T, st2, cs2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(st, st2)


def test_long_prefill_chained_equals_single_shot():
    wl = I.WORKLOADS["long_prefill_t32768"]
    say("case long_prefill_t32768: 8 chained calls of 4096 vs one call, oracle on 8 heads")
    inp = I.generate(wl)
    layer = TT.make_layer(wl, inp, DEV)
    st, cs = _dev_state(wl, inp)
    step = wl.T // wl.splits
    outs = []
    for i in range(wl.splits):
        outs.append(_gpu_prefill(wl, inp, layer, i * step, (i + 1) * step, st, cs))
    chained = torch.cat(outs, dim=1)
    del outs
    st1, cs1 = _dev_state(wl, inp)
    single = _gpu_prefill(wl, inp, layer, 0, wl.T, st1, cs1)
    torch.cuda.synchronize()
    _check("chained vs single out", chained, TT.to_host_f64(single), TOL["bf16"])
    _check("chained vs single state", st, TT.to_host_f64(st1), TOL["bf16"])
    assert torch.equal(cs, cs1)
    heads = [0, 5, 9, 14, 18, 23, 27, 31]
    swl, sinp = I.select_heads(wl, inp, heads)
    ref = oracle_layer(swl, sinp, 0, wl.T, sinp["state0"], sinp["conv_state0"])
    oc, ch = head_channels(wl, heads)
    _check("chained out (8 heads)", chained[..., oc], ref["out"], TOL["bf16"])
    _check("chained state (8 heads)", st[:, heads], ref["state"], TOL["bf16"])
    _check("single-shot out (8 heads)", single[..., oc], ref["out"], TOL["bf16"])
    _check("chained conv_state (8 heads)", cs[:, ch], ref["conv_state"], 0.0)


# ---------------------------------------------------------------------------
# Input projection ahead of the layer
# ---------------------------------------------------------------------------

def _gpu_projection(wl, inp, out_dtype, rows=None):
    ot = abi.KDA_BF16 if out_dtype == torch.bfloat16 else abi.KDA_F32
    dev = {k: TT.to_device(v, "bf16", DEV) for k, v in inp.items()}
    proj = abi.KdaProjection(H=wl.H, D=wl.d, hidden=wl.hidden, rank=wl.rank, out_dtype=ot, w_in=dev["w_in"],
                             w_fb=dev["w_fb"], w_gb=dev["w_gb"])
    HD = wl.H * wl.d
    out = {"qkv": torch.empty((wl.T, 3 * HD), dtype=out_dtype, device=DEV),
           "f": torch.empty((wl.T, HD), dtype=out_dtype, device=DEV),
           "beta": torch.empty((wl.T, wl.H), dtype=out_dtype, device=DEV),
           "g_out": torch.empty((wl.T, HD), dtype=out_dtype, device=DEV)}
    ws = torch.empty(abi.kda_input_projection_workspace_size(proj, wl.T), dtype=torch.uint8, device=DEV)
    abi.kda_input_projection(proj, dev["x"], out["qkv"], out["f"], out["beta"], out["g_out"], ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("T", [100, 1, 64])
def test_input_projection_small(T):
    from dataclasses import replace
    wl = replace(I.PROJ_WORKLOADS["projection_t4096"], T=T, hidden=256, H=4, seed=60 + T)
    say(f"case input projection T={T} hidden=256 H=4 d=128 rank=128")
    inp = I.generate_projection(wl)
    ref = O.kda_input_projection(inp["x"], inp["w_in"], inp["w_fb"], inp["w_gb"], wl.H, wl.d, wl.rank)
    out = _gpu_projection(wl, inp, torch.float32)
    for k in ("qkv", "f", "beta", "g_out"):
        _check(k, out[k], ref[k], TOL["bf16"])
    out16 = _gpu_projection(wl, inp, torch.bfloat16)
    for k in ("qkv", "f", "beta", "g_out"):
        _check(f"{k} (bf16 output)", out16[k], ref[k], TOL_BF16_OUT)


def test_input_projection_full_size_sampled_rows():
    wl = I.PROJ_WORKLOADS["projection_t4096"]
    say("case input projection full size (T=4096, hidden=4096, H=32, d=128, rank=128), 48 sampled rows")
    inp = I.generate_projection(wl)
    out = _gpu_projection(wl, inp, torch.float32)
    rows = np.random.default_rng(0).choice(wl.T, 48, replace=False)
    ref = O.kda_input_projection(inp["x"][rows], inp["w_in"], inp["w_fb"], inp["w_gb"], wl.H, wl.d, wl.rank)
    idx = torch.from_numpy(rows).to(DEV)
    for k in ("qkv", "f", "beta", "g_out"):
        _check(k, out[k].index_select(0, idx), ref[k], TOL["bf16"])
