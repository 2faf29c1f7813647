"""Benchmark of the KDA layer hot path on one MI355X.

One step = one pass over every call of the path on its layer-shaped workload:
  prefill   B=1, T=4096, H=32, d_k=d_v=128, chunk 64, bf16 io, fp32 state
  decode    64 sequences x 32 heads x 128x128 fp32 state, one token each
  verify    16 sequences x 8 draft tokens with per-token snapshots, then rollback
            to a seeded accepted prefix (0..8) per sequence
Inputs are seeded synthetic tensors (hybrid_linear_attention_kda_amd.inputs);
the decode / verify states are pre-filled on the GPU by running 256 / 2048
random tokens through kda_prefill first.  Every call rotates over --sets
independent buffer sets (default 4, > 2x the 256 MB Infinity Cache per
call type), so timed bytes come from HBM.

Prints ONE JSON line: value = prefill tokens/s; the decode state-update GB/s,
verify GB/s and per-call times ride along; `roofline` is for the dominant
kernel, `cpu_baseline` times the float64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_bytes(B, T, H, D, W, io_b=2, out_b=2):
    per_tok = (3 * H * D + H * D + H * D) * io_b + H * io_b + H * D * out_b  # qkv, f, g_out, beta, out
    state = 2 * B * H * D * D * 4
    conv = 2 * B * 3 * H * D * (W - 1) * io_b
    params = 3 * H * D * W * io_b + H * 4 + H * D * 4 + D * io_b
    return B * T * per_tok + state + conv + params


def decode_bytes(B, H, D, W, io_b=2, out_b=2):
    return prefill_bytes(B, 1, H, D, W, io_b, out_b)


def verify_bytes(B, T_d, H, D, W, io_b=2, out_b=2):
    per_tok = (3 * H * D + H * D + H * D) * io_b + H * io_b + H * D * out_b
    state_read = B * H * D * D * 4
    snaps = B * T_d * H * D * D * 4
    conv = B * 3 * H * D * (W - 1) * io_b
    params = 3 * H * D * W * io_b + H * 4 + H * D * 4 + D * io_b
    return B * T_d * per_tok + state_read + snaps + conv + params


def rollback_bytes(accepted, H, D, W, io_b=2):
    n = sum(1 for m in accepted if m > 0)
    return n * (2 * H * D * D * 4 + 2 * 3 * H * D * (W - 1) * io_b) + sum(int(m) for m in accepted) * 0


def cpu_baseline(sample_heads: int, T: int):
    """The float64 oracle, as it stands, on a bounded sample of the prefill workload:
    `sample_heads` of the 32 heads over T tokens (heads are independent, so the
    full layer costs 32 / sample_heads times as much)."""
    from threadpoolctl import threadpool_limits

    from hybrid_linear_attention_kda_amd import inputs as I
    from oracle import kda_oracle as O

    wl = I.WORKLOADS["prefill_t4096"].with_(T=T)
    inp = I.generate(wl)
    heads = list(range(sample_heads))
    swl, sinp = I.select_heads(wl, inp, heads)
    p = O.KdaParams(H=swl.H, dk=swl.dk, dv=swl.dv, conv_w=sinp["conv_w"], A_log=sinp["A_log"],
                    dt_bias=sinp["dt_bias"], norm_w=sinp["norm_w"], lb=sinp["lb"], scale=sinp["scale"])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.kda_layer(p, sinp["qkv"], sinp["f"], sinp["beta"], sinp["g_out"], sinp["state0"], sinp["conv_state0"])
        dt = time.perf_counter() - t0
    full_layer_s = dt * wl.H / sample_heads
    return {"value": T / full_layer_s, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 token-recurrence oracle, {sample_heads} of 32 heads x {T} tokens of the "
                      f"T=4096 prefill workload ({dt:.1f} s), scaled to 32 heads; BLAS limited to 1 thread"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--only", choices=["prefill", "decode", "verify"], default=None,
                    help="time one call type only (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=4)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards by head with "
              f"no communication, so per-GPU throughput at N GPUs is the single-GPU figure at H/N heads.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from hybrid_linear_attention_kda_amd import abi
    from hybrid_linear_attention_kda_amd import inputs as I
    from hybrid_linear_attention_kda_amd import tensors as TT

    dev = "cuda:0"
    torch.cuda.set_device(0)
    abi.load()
    stream = torch.cuda.current_stream()
    nsets = max(1, args.sets)

    wp, wd, wv = I.WORKLOADS["prefill_t4096"], I.WORKLOADS["decode_b64"], I.WORKLOADS["verify_b16"]
    ops = ["prefill", "decode", "verify"] if args.only is None else [args.only]

    def workspace(layer, B, T):
        n = abi.kda_prefill_workspace_size(layer, B, T)
        return torch.empty(n, dtype=torch.uint8, device=dev) if n else None

    sets = {op: [] for op in ops}
    # --- prefill sets
    if "prefill" in ops:
        inp = I.generate(wp)
        lay = TT.make_layer(wp, inp, dev, out="bf16")
        tok = TT.token_tensors(wp, inp, 0, wp.T, dev)
        for _ in range(nsets):
            sets["prefill"].append(dict(
                layer=lay, tok={k: v.clone() for k, v in tok.items()},
                state=torch.zeros((1, wp.H, wp.dk, wp.dv), dtype=torch.float32, device=dev),
                conv=torch.zeros((1, wp.c_qkv, wp.W - 1), dtype=torch.bfloat16, device=dev),
                out=torch.empty((1, wp.T, wp.H * wp.dv), dtype=torch.bfloat16, device=dev),
                ws=workspace(lay, 1, wp.T)))
        del tok

    def prefilled(wl, inp, lay):
        pre = TT.token_tensors(wl, inp, 0, wl.prefix_T, dev)
        st = torch.zeros((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        cs = torch.zeros((wl.B, wl.c_qkv, wl.W - 1), dtype=torch.bfloat16, device=dev)
        o = torch.empty((wl.B, wl.prefix_T, wl.H * wl.dv), dtype=torch.bfloat16, device=dev)
        abi.kda_prefill(lay, pre["qkv"], pre["f"], pre["beta"], pre["g_out"], st, cs, o,
                        workspace=workspace(lay, wl.B, wl.prefix_T))
        torch.cuda.synchronize()
        return st, cs

    if "decode" in ops:
        inp = I.generate(wd)
        lay = TT.make_layer(wd, inp, dev, out="bf16")
        st, cs = prefilled(wd, inp, lay)
        tok = TT.token_tensors(wd, inp, wd.prefix_T, wd.prefix_T + 1, dev)
        for _ in range(nsets):
            sets["decode"].append(dict(layer=lay, tok={k: v.clone() for k, v in tok.items()}, state=st.clone(),
                                       conv=cs.clone(),
                                       out=torch.empty((wd.B, 1, wd.H * wd.dv), dtype=torch.bfloat16, device=dev)))
        del st, cs
    accepted = None
    if "verify" in ops:
        inp = I.generate(wv)
        accepted = [int(m) for m in inp["accepted"]]
        lay = TT.make_layer(wv, inp, dev, out="bf16")
        st, cs = prefilled(wv, inp, lay)
        tok = TT.token_tensors(wv, inp, wv.prefix_T, wv.prefix_T + wv.T, dev)
        for _ in range(nsets):
            sets["verify"].append(dict(
                layer=lay, tok={k: v.clone() for k, v in tok.items()}, state=st.clone(), conv=cs.clone(),
                snaps=torch.empty((wv.B, wv.T, wv.H, wv.dk, wv.dv), dtype=torch.float32, device=dev),
                out=torch.empty((wv.B, wv.T, wv.H * wv.dv), dtype=torch.bfloat16, device=dev)))
        del st, cs
    torch.cuda.synchronize()

    def run(op, s):
        t = s["tok"]
        if op == "prefill":
            abi.kda_prefill(s["layer"], t["qkv"], t["f"], t["beta"], t["g_out"], s["state"], s["conv"], s["out"],
                            workspace=s["ws"], stream=stream)
        elif op == "decode":
            abi.kda_decode_step(s["layer"], t["qkv"], t["f"], t["beta"], t["g_out"], s["state"], s["conv"],
                                s["out"], stream=stream)
        elif op == "verify":
            abi.kda_verify_block(s["layer"], t["qkv"], t["f"], t["beta"], t["g_out"], s["state"], s["conv"],
                                 s["snaps"], s["out"], stream=stream)
        elif op == "rollback":
            abi.kda_rollback(s["layer"], accepted, s["snaps"], t["qkv"], s["state"], s["conv"], stream=stream)

    seq = []
    for op in ops:
        seq.append(op)
        if op == "verify":
            seq.append("rollback")

    def setof(op):
        return "verify" if op == "rollback" else op

    for i in range(args.warmup):
        for op in seq:
            run(op, sets[setof(op)][i % nsets])
    torch.cuda.synchronize()

    K = args.steps
    ev = {op: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
          for op in seq}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        for op in seq:
            e0, e1 = ev[op][i]
            e0.record(stream)
            run(op, sets[setof(op)][i % nsets])
            e1.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms = {op: np.array([a.elapsed_time(b) for a, b in ev[op]]) for op in seq}
    mean = {op: float(ms[op].mean()) for op in seq}
    med = {op: float(np.median(ms[op])) for op in seq}

    res = {
        "metric": "KDA prefill tokens/s (H=32,128x128,T=4096) + decode state-update HBM GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_total / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_t4096 (B=1,T=4096,H=32,d=128,chunk 64) + decode_b64 (B=64,H=32,d=128) + "
                               "verify_b16 (B=16,T_d=8,H=32,d=128) with rollback",
                   "io": "bf16 inputs and outputs, fp32 state and accumulation", "buffer_sets": nsets},
        "wall_s": wall,
    }
    detail = {}
    roof_candidates = []
    if "prefill" in ops:
        pb = prefill_bytes(1, wp.T, wp.H, wp.dk, wp.W)
        res["value"] = wp.T / (mean["prefill"] * 1e-3)
        res["unit"] = "tokens/s"
        detail["prefill"] = {"ms_mean": mean["prefill"], "ms_median": med["prefill"],
                             "ms_p10": float(np.percentile(ms["prefill"], 10)),
                             "ms_p90": float(np.percentile(ms["prefill"], 90)),
                             "tokens_per_s": res["value"], "alg_bytes": pb,
                             "gbps": pb / (mean["prefill"] * 1e-3) / 1e9}
        roof_candidates.append(("prefill", mean["prefill"], pb))
    if "decode" in ops:
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.W)
        gb = db / (mean["decode"] * 1e-3) / 1e9
        res["decode_state_update_gbps"] = gb
        detail["decode"] = {"ms_mean": mean["decode"], "ms_median": med["decode"], "alg_bytes": db, "gbps": gb,
                            "hbm_frac": gb / HBM_PEAK_GBPS}
        roof_candidates.append(("decode", mean["decode"], db))
        if "value" not in res:
            res["value"], res["unit"] = gb, "GB/s"
    if "verify" in ops:
        vb = verify_bytes(wv.B, wv.T, wv.H, wv.dk, wv.W)
        rb = rollback_bytes(accepted, wv.H, wv.dk, wv.W)
        gv = vb / (mean["verify"] * 1e-3) / 1e9
        detail["verify"] = {"ms_mean": mean["verify"], "ms_median": med["verify"], "alg_bytes": vb, "gbps": gv,
                            "hbm_frac": gv / HBM_PEAK_GBPS}
        detail["rollback"] = {"ms_mean": mean["rollback"], "alg_bytes": rb,
                              "gbps": rb / (mean["rollback"] * 1e-3) / 1e9, "accepted": accepted}
        roof_candidates.append(("verify", mean["verify"], vb))
        if "value" not in res:
            res["value"], res["unit"] = gv, "GB/s"
    res["detail"] = detail
    # dominant kernel: the call with the largest share of the step
    name, t_ms, nbytes = max(roof_candidates, key=lambda c: c[1])
    achieved = nbytes / (t_ms * 1e-3) / 1e9
    res["roofline"] = {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": None}
    if not args.no_cpu_baseline and "prefill" in ops:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(args.cpu_heads, wp.T)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
