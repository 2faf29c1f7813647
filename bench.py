"""Benchmark of the KDA layer hot path on one MI355X.

One step = one pass over every call of the path on its layer-shaped workload:
  prefill   B=1, T=4096, H=32, d_k=d_v=128, chunk 64, bf16 io, fp32 state
  varlen    the same 4096 tokens as 16 packed sequences of a seeded length mix
            (123..628 tokens), each from its own zero state slot
  decode    64 sequences x 32 heads x 128x128 fp32 state, one token each
  softplus  prefill_t4096 and decode_b64 again with the softplus decay branch (no lower bound)
  strong    prefill_t4096 again with the bounded gate at gate_lower_bound = -8 (below the range of
            start-anchored sub-chunks: end-anchored ones with exact diagonal blocks)
  projection  the layer's input projection for those 4096 tokens: hidden 4096 -> q|k|v, f, beta,
            g_out (H=32, d=128, rank 128; the q|k|v|f_a|g_a|b projections as one matmul)
  verify    16 sequences x 8 draft tokens with per-token snapshots, then rollback
            to a seeded accepted prefix (0..8) per sequence; and the same block
            verified with a replay tape, then committed from the tape
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
    return n * (2 * H * D * D * 4 + 2 * 3 * H * D * (W - 1) * io_b)


def verify_tape_bytes(B, T_d, H, D, W, io_b=2, out_b=2):
    """verify with a replay tape: the snapshots are replaced by 3*D floats per token and head"""
    return verify_bytes(B, T_d, H, D, W, io_b, out_b) - B * T_d * H * D * D * 4 + B * T_d * H * 3 * D * 4


def commit_bytes(accepted, H, D, W, io_b=2):
    """tape commit: the state of every sequence with m > 0 read and written, its m tape rows read"""
    return rollback_bytes(accepted, H, D, W, io_b) + sum(int(m) for m in accepted) * H * 3 * D * 4


VARLEN_SEQS = 16
VARLEN_SEED = 8


def kernel_alg_bytes(kernel, wp, wd, wv, accepted):
    """Algorithmic bytes of one launch of each kernel: what the launch must read and write once,
    with the prefill call's bytes split over its four kernels (their sum is prefill_bytes)."""
    io_b = 2
    Hp, Dp, Wp, Tp = wp.H, wp.dk, wp.W, wp.T
    params = 3 * Hp * Dp * Wp * io_b + Hp * 4 + Hp * Dp * 4
    conv = 3 * Hp * Dp * (Wp - 1) * io_b
    table = {
        # qkv, f, beta of every token, the conv state in, conv weights, A_log, dt_bias
        "kda_chunk_prep_kernel": Tp * (3 * Hp * Dp * io_b + Hp * Dp * io_b + Hp * io_b) + conv + params,
        # fp32 state in and out, conv state out
        "kda_chunk_state_kernel": 2 * Hp * Dp * Dp * 4 + conv,
        # g_out in, out written, norm weight
        "kda_out_norm_kernel": Tp * 2 * Hp * Dp * io_b + Dp * io_b,
        # the variable-length call: the same tokens, a state and conv state per sequence
        "kda_chunk_prep_kernel[varlen]": Tp * (3 * Hp * Dp * io_b + Hp * Dp * io_b + Hp * io_b)
                                         + VARLEN_SEQS * conv + params,
        "kda_chunk_state_kernel[varlen]": VARLEN_SEQS * (2 * Hp * Dp * Dp * 4 + conv),
        "kda_out_norm_kernel[varlen]": Tp * 2 * Hp * Dp * io_b + Dp * io_b,
        "kda_recurrent_kernel[decode]": decode_bytes(wd.B, wd.H, wd.dk, wd.W),
        "kda_recurrent_kernel[decode][softplus]": decode_bytes(wd.B, wd.H, wd.dk, wd.W),
        "kda_recurrent_kernel[verify]": verify_bytes(wv.B, wv.T, wv.H, wv.dk, wv.W),
        "kda_rollback_kernel": rollback_bytes(accepted or [], wv.H, wv.dk, wv.W),
        "kda_recurrent_kernel[verify_tape]": verify_tape_bytes(wv.B, wv.T, wv.H, wv.dk, wv.W),
        "kda_commit_tape_kernel": commit_bytes(accepted or [], wv.H, wv.dk, wv.W),
    }
    for k in ("kda_chunk_prep_kernel", "kda_chunk_state_kernel", "kda_out_norm_kernel"):
        table[k + "[softplus]"] = table[k]  # the softplus decay branch: the same bytes
        table[k + "[strong]"] = table[k]    # the bounded gate below -5.5: the same bytes
    return table.get(kernel)


def source_fingerprint():
    """sha256 over the HIP sources and headers of the library: counter-derived traffic is only
    reported while the kernels are the ones it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "hybrid_linear_attention_kda_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
CALIB_BYTES = 384 << 20  # the plain copy kernel of --calib-copy reads and writes this many bytes


def stored_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter runs, or None when there are
    none for it or the sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("source_sha256") != source_fingerprint():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None:
        return None
    return k["fetch_bytes"] + k["write_bytes"]


def projection_flops(wl):
    """useful flops of one input projection: the fused GEMM and the two rank-r up-projections"""
    HD = wl.H * wl.d
    return 2 * wl.T * wl.hidden * (3 * HD + 2 * wl.rank + wl.H) + 2 * 2 * wl.T * wl.rank * HD


def kernel_alg_flops(kernel, wj):
    """Useful flops of one launch of the input projection's kernels (matrix-core bound, no bytes)."""
    HD = wj.H * wj.d
    return {"kda_proj_gemm_kernel": 2 * wj.T * wj.hidden * (3 * HD + 2 * wj.rank + wj.H),
            "kda_proj_lowrank_kernel": 2 * 2 * wj.T * wj.rank * HD}.get(kernel)


def short_kernel_name(full):
    import re
    m = re.search(r"(kda_[a-z0-9_]+_kernel)(<[^>]*>)?", full)
    if m is None:
        return None
    name = m.group(1)
    if name == "kda_chunk_state64_kernel":  # the uniform-batch state pass (the library's timing name)
        name = "kda_chunk_state_kernel"
    targs = m.group(2) or ""
    if not targs:
        # a name the profiler left mangled: template arguments as ILb<0|1>E[Li<n>E]...
        mm = re.match(re.escape(m.group(1)) + r"I(Lb([01])E)(Li(\d+)E)?", full[m.start(1):])
        if mm:
            targs = "<" + ("true" if mm.group(2) == "1" else "false") + (", " + mm.group(4) if mm.group(4) else "") + ">"
    if name in ("kda_chunk_prep_kernel", "kda_chunk_state_kernel") and targs.startswith("<true"):
        name += "[varlen]"
    if name == "kda_chunk_prep_kernel":
        gk = targs.rstrip(">").split(",")[-1].strip()
        name += {"1": "[softplus]", "2": "[strong]"}.get(gk, "")
    if name == "kda_recurrent_kernel" and m.group(2):
        targs = m.group(2)
        name += "[verify_tape]" if ", true, true," in targs else "[verify]" if ", true," in targs else "[decode]"
    return name


def pmc_summary(fetch_dir, write_dir, command):
    """Scale the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch) of two rocprofv3 --pmc runs
    of `bench.py ... --calib-copy` by what they read for the plain copy kernel of CALIB_BYTES,
    and store bytes per launch per kernel in profiles/pmc_traffic.json."""
    import csv
    import glob

    def per_kernel(d, counter):
        acc = {}
        calib = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0
                name = short_kernel_name(r["Kernel_Name"])
                if name is not None:
                    acc.setdefault(name, []).append(v)
                elif "neg_kernel" in r["Kernel_Name"]:
                    calib.append(v)
        return acc, calib

    fetch, fcal = per_kernel(fetch_dir, "FETCH_SIZE")
    write, wcal = per_kernel(write_dir, "WRITE_SIZE")
    # the calibration copy is torch's neg over CALIB_BYTES (the only neg launch of the run)
    fc = max(fcal) / CALIB_BYTES
    wc = max(wcal) / CALIB_BYTES
    out = {"command": command, "source_sha256": source_fingerprint(),
           "calibration": {"copy_bytes": CALIB_BYTES, "fetch_factor": fc, "write_factor": wc},
           "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        f = float(np.mean(fetch.get(k, [0.0]))) / fc
        w = float(np.mean(write.get(k, [0.0]))) / wc
        out["kernels"][k] = {"fetch_bytes": f, "write_bytes": w, "dispatches": len(fetch.get(k, []))}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))


def mfma_summary(pmc_dir, command, n_cu=256):
    """Per-kernel instruction counts from one rocprofv3 --pmc run of the SQ counters (SQ_INSTS_MFMA,
    SQ_INSTS_VALU, SQ_INSTS_LDS, ...): the mean over the kernel's dispatches, and the issued matrix-core
    rate, SQ_INSTS_MFMA x 16,384 flop (one 16x16x32 bf16 / fp16 product; the few fp32 16x16x4 steps of
    the prefill count the same, an upper bound) over the dispatch's duration, as a fraction of the dense
    bf16 peak; stored in profiles/pmc_mfma.json with the sources' sha256."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            name = short_kernel_name(r["Kernel_Name"])
            if name is None:
                continue
            key = (name, r.get("Dispatch_Id", r.get("Correlation_Id", "")))
            rec = vals.setdefault(name, {}).setdefault(key, {})
            rec[r["Counter_Name"]] = float(r["Counter_Value"])
            rec["duration_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    out = {"command": command, "source_sha256": source_fingerprint(), "n_cu": n_cu, "kernels": {}}
    for name, disp in sorted(vals.items()):
        fr, mf, va, ld = [], [], [], []
        for c in disp.values():
            if "SQ_INSTS_MFMA" in c and c["duration_ns"] > 0:
                fr.append(c["SQ_INSTS_MFMA"] * 16384 / (c["duration_ns"] * 1e-9) / 1e12 / BF16_MFMA_PEAK_TFLOPS)
            if "SQ_INSTS_MFMA" in c:
                mf.append(c["SQ_INSTS_MFMA"])
            if "SQ_INSTS_VALU" in c:
                va.append(c["SQ_INSTS_VALU"])
            if "SQ_INSTS_LDS" in c:
                ld.append(c["SQ_INSTS_LDS"])
        out["kernels"][name] = {"mfma_issued_frac": float(np.mean(fr)) if fr else None,
                                "insts_mfma": float(np.mean(mf)) if mf else None,
                                "insts_valu": float(np.mean(va)) if va else None,
                                "insts_lds": float(np.mean(ld)) if ld else None, "dispatches": len(disp)}
    json.dump(out, open(SQ_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(sample_heads: int, T: int, chunked_heads: int = 8):
    """The float64 oracle, as it stands, on a bounded sample of the prefill workload, with its BLAS
    on every host core this process may use: the token recurrence (the definition) on
    `sample_heads` of the 32 heads over T tokens, and the chunked WY/UT spelling on `chunked_heads`
    heads (heads are independent, so the full layer costs 32 / heads times as much)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from hybrid_linear_attention_kda_amd import inputs as I
    from oracle import kda_oracle as O

    cores = len(os.sched_getaffinity(0))
    wl = I.WORKLOADS["prefill_t4096"].with_(T=T)
    inp = I.generate(wl)

    def run(nh, form):
        swl, sinp = I.select_heads(wl, inp, list(range(nh)))
        p = O.KdaParams(H=swl.H, dk=swl.dk, dv=swl.dv, conv_w=sinp["conv_w"], A_log=sinp["A_log"],
                        dt_bias=sinp["dt_bias"], norm_w=sinp["norm_w"], lb=sinp["lb"], scale=sinp["scale"])
        t0 = time.perf_counter()
        O.kda_layer(p, sinp["qkv"], sinp["f"], sinp["beta"], sinp["g_out"], sinp["state0"], sinp["conv_state0"],
                    form=form, chunk=wl.chunk)
        return time.perf_counter() - t0

    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        dt_tok = run(sample_heads, "token")
        dt_chk = run(chunked_heads, "chunked")
    tok_s = T / (dt_tok * wl.H / sample_heads)
    chk_s = T / (dt_chk * wl.H / chunked_heads)
    return {"value": tok_s, "unit": "tokens/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": f"float64 token-recurrence oracle, {sample_heads} of 32 heads x {T} tokens of the T=4096 "
                      f"prefill workload ({dt_tok:.1f} s), scaled to 32 heads; BLAS on {min(cores, threads)} "
                      f"threads ({cores} cores in this process's affinity mask)",
            "chunked": {"value": chk_s, "unit": "tokens/s",
                        "sample": f"float64 chunked WY/UT oracle (chunk 64), {chunked_heads} of 32 heads x {T} "
                                  f"tokens ({dt_chk:.1f} s), scaled to 32 heads"}}


PREFILL_CHUNK = 64


def prefill_alg_flops(T, H, D, C=PREFILL_CHUNK):
    """Algorithmic flops of one chunked prefill call, dense tiles (triangular products counted whole):
    per chunk-head A_kk, A_qk, W = T X, Ut = T (beta V) and A_qk U (2 C^2 D each), the UT inverse
    (C^3 / 3 x 2) and the three products with the state U = Ut - W S, Q~ S, K~^T U (2 C D^2 each)."""
    nch = (T + C - 1) // C
    per = 5 * 2 * C * C * D + 2 * C ** 3 // 3 + 3 * 2 * C * D * D
    return nch * H * per


SQ_FILE = os.path.join(ROOT, "profiles", "pmc_mfma.json")


def stored_mfma_issued(kernel):
    """Issued matrix-core rate of `kernel` as a fraction of the dense bf16 peak from the committed
    counter run (SQ_INSTS_MFMA x 16,384 flop over the dispatch time), or None when there is none or
    the sources changed since."""
    if not os.path.exists(SQ_FILE):
        return None
    rec = json.load(open(SQ_FILE))
    if rec.get("source_sha256") != source_fingerprint():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("mfma_issued_frac")


def hbm_ceilings(dev, nbytes=1 << 30, reps=5):
    """Measured HBM ceilings on this GPU, each the median of `reps` runs on buffers well beyond the
    256 MB last-level cache: a plain copy (nbytes read + nbytes written) and a write-only fill, each
    by torch (copy_, fill_) and by the library's streaming copy (kda_measure_stream: 16-byte
    non-temporal accesses, four loads in flight per lane), and a read-only reduction (torch sum, a
    few bytes out).  "copy" and "write" are the higher of the two."""
    import torch
    from hybrid_linear_attention_kda_amd import abi
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("copy_torch", lambda: dst.copy_(src), 2 * nbytes),
                            ("copy_stream", lambda: abi.measure_stream(dst, src), 2 * nbytes),
                            ("write_torch", lambda: dst.fill_(2.0), nbytes),
                            ("write_stream", lambda: abi.measure_stream(dst), nbytes),
                            ("read", lambda: src.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        out[name] = {"gbps": moved / (ms * 1e-3) / 1e9, "bytes": moved, "ms_median": ms}
    for k in ("copy", "write"):
        out[k] = max(out[k + "_torch"], out[k + "_stream"], key=lambda r: r["gbps"])
    del src, dst
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--only", choices=["prefill", "varlen", "projection", "decode", "verify"], default=None,
                    help="time one call type only (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=32)
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run one plain copy kernel of known size (for counter scaling)")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "COMMAND"),
                    help="turn two rocprofv3 --pmc runs into profiles/pmc_traffic.json and exit")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("PMC_DIR", "COMMAND"),
                    help="turn a rocprofv3 --pmc run of the matrix-core counters into profiles/pmc_mfma.json and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.mfma_summary:
        mfma_summary(*args.mfma_summary)
        return
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
    wf, wt = wp.with_(T=1024, io="f32"), I.WORKLOADS["tiny_fp32"]
    ops = ["prefill", "varlen", "projection", "decode", "verify"] if args.only is None else [args.only]

    def strong_layer(lay):
        """The same layer parameters with the bounded gate at gate_lower_bound = -8."""
        return abi.KdaLayer(H=lay.H, D=lay.D, W=lay.W, chunk=lay.chunk, io_dtype=lay.io_dtype,
                            out_dtype=lay.out_dtype, lb=-8.0, scale=lay.scale, conv_w=lay.conv_w,
                            A_log=lay.A_log, dt_bias=lay.dt_bias, norm_w=lay.norm_w)

    def softplus_layer(lay):
        """The same layer parameters on the softplus decay branch (no lower bound)."""
        return abi.KdaLayer(H=lay.H, D=lay.D, W=lay.W, chunk=lay.chunk, io_dtype=lay.io_dtype,
                            out_dtype=lay.out_dtype, lb=float("nan"), scale=lay.scale, conv_w=lay.conv_w,
                            A_log=lay.A_log, dt_bias=lay.dt_bias, norm_w=lay.norm_w,
                            gate_kind=abi.KDA_GATE_SOFTPLUS)

    def workspace(layer, B, T):
        n = abi.kda_prefill_workspace_size(layer, B, T)
        return torch.empty(n, dtype=torch.uint8, device=dev) if n else None

    sets = {op: [] for op in ops}
    # --- prefill sets
    if "prefill" in ops:
        inp = I.generate(wp)
        lay = TT.make_layer(wp, inp, dev, out="bf16")
        tok = TT.token_tensors(wp, inp, 0, wp.T, dev)
        lay_sp = softplus_layer(lay)
        lay_st = strong_layer(lay)
        for _ in range(nsets):
            sets["prefill"].append(dict(
                layer=lay, layer_sp=lay_sp, layer_st=lay_st, tok={k: v.clone() for k, v in tok.items()},
                state=torch.zeros((1, wp.H, wp.dk, wp.dv), dtype=torch.float32, device=dev),
                conv=torch.zeros((1, wp.c_qkv, wp.W - 1), dtype=torch.bfloat16, device=dev),
                out=torch.empty((1, wp.T, wp.H * wp.dv), dtype=torch.bfloat16, device=dev),
                ws=workspace(lay, 1, wp.T)))
        del tok
        # the fp32 vector-ALU prefill (fp32 io and out) on a 1024-token cut of the same layer shape,
        # and the small fp32 layer (B=1, T=64, H=2, d=16, chunk 16) through the same path
        for key, wl in (("prefill_f32", wf), ("prefill_tiny", wt)):
            inp = I.generate(wl)
            lay = TT.make_layer(wl, inp, dev, out="f32")
            tok = TT.token_tensors(wl, inp, 0, wl.T, dev)
            sets[key] = [dict(layer=lay, tok={k: v.clone() for k, v in tok.items()},
                              state=torch.zeros((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev),
                              conv=torch.zeros((wl.B, wl.c_qkv, wl.W - 1), dtype=torch.float32, device=dev),
                              out=torch.empty((wl.B, wl.T, wl.H * wl.dv), dtype=torch.float32, device=dev),
                              ws=workspace(lay, wl.B, wl.T)) for _ in range(nsets)]
            del tok
    # --- variable-length sets: the prefill tokens as packed sequences of a seeded length mix
    var_lens = I.varlen_lengths(wp.T, VARLEN_SEQS, VARLEN_SEED)
    var_cu = I.cu_seqlens(var_lens)
    if "varlen" in ops:
        inp = I.generate(wp)
        lay = TT.make_layer(wp, inp, dev, out="bf16")
        tok = TT.token_tensors(wp, inp, 0, wp.T, dev)
        nvs = abi.kda_prefill_varlen_workspace_size(lay, var_cu)
        for _ in range(nsets):
            sets["varlen"].append(dict(
                layer=lay, tok={k: v[0].clone() for k, v in tok.items()},
                state=torch.zeros((VARLEN_SEQS, wp.H, wp.dk, wp.dv), dtype=torch.float32, device=dev),
                conv=torch.zeros((VARLEN_SEQS, wp.c_qkv, wp.W - 1), dtype=torch.bfloat16, device=dev),
                out=torch.empty((wp.T, wp.H * wp.dv), dtype=torch.bfloat16, device=dev),
                ws=torch.empty(nvs, dtype=torch.uint8, device=dev)))
        del tok

    wj = I.PROJ_WORKLOADS["projection_t4096"]
    if "projection" in ops:
        pin = I.generate_projection(wj)
        HDj = wj.H * wj.d
        pw = {k: TT.to_device(pin[k], "bf16", dev) for k in ("w_in", "w_fb", "w_gb")}
        proj = abi.KdaProjection(H=wj.H, D=wj.d, hidden=wj.hidden, rank=wj.rank, out_dtype=abi.KDA_BF16, **pw)
        x = TT.to_device(pin["x"], "bf16", dev)
        npw = abi.kda_input_projection_workspace_size(proj, wj.T)
        for _ in range(nsets):
            sets["projection"].append(dict(
                proj=proj, x=x.clone(),
                qkv=torch.empty((wj.T, 3 * HDj), dtype=torch.bfloat16, device=dev),
                f=torch.empty((wj.T, HDj), dtype=torch.bfloat16, device=dev),
                beta=torch.empty((wj.T, wj.H), dtype=torch.bfloat16, device=dev),
                g=torch.empty((wj.T, HDj), dtype=torch.bfloat16, device=dev),
                ws=torch.empty(npw, dtype=torch.uint8, device=dev)))
        del pin, x

    def prefilled(wl, inp):
        # The prefix runs through the fp32-io prefill (its own kernel, the inputs are bf16 values
        # held exactly in fp32), so the timed kernels' launches are all of the timed shapes.
        w32 = wl.with_(io="f32")
        lay32 = TT.make_layer(w32, inp, dev, out="f32")
        pre = TT.token_tensors(w32, inp, 0, wl.prefix_T, dev)
        st = torch.zeros((wl.B, wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        cs = torch.zeros((wl.B, wl.c_qkv, wl.W - 1), dtype=torch.float32, device=dev)
        o = torch.empty((wl.B, wl.prefix_T, wl.H * wl.dv), dtype=torch.float32, device=dev)
        abi.kda_prefill(lay32, pre["qkv"], pre["f"], pre["beta"], pre["g_out"], st, cs, o,
                        workspace=workspace(lay32, wl.B, wl.prefix_T))
        torch.cuda.synchronize()
        return st, cs.to(torch.bfloat16)

    if "decode" in ops:
        inp = I.generate(wd)
        lay = TT.make_layer(wd, inp, dev, out="bf16")
        st, cs = prefilled(wd, inp)
        tok = TT.token_tensors(wd, inp, wd.prefix_T, wd.prefix_T + 1, dev)
        lay_sp = softplus_layer(lay)
        for _ in range(nsets):
            sets["decode"].append(dict(layer=lay, layer_sp=lay_sp, tok={k: v.clone() for k, v in tok.items()},
                                       state=st.clone(),
                                       conv=cs.clone(),
                                       out=torch.empty((wd.B, 1, wd.H * wd.dv), dtype=torch.bfloat16, device=dev)))
        del st, cs
    accepted = None
    if "verify" in ops:
        inp = I.generate(wv)
        accepted = [int(m) for m in inp["accepted"]]
        lay = TT.make_layer(wv, inp, dev, out="bf16")
        st, cs = prefilled(wv, inp)
        tok = TT.token_tensors(wv, inp, wv.prefix_T, wv.prefix_T + wv.T, dev)
        for _ in range(nsets):
            sets["verify"].append(dict(
                layer=lay, tok={k: v.clone() for k, v in tok.items()}, state=st.clone(), conv=cs.clone(),
                snaps=torch.empty((wv.B, wv.T, wv.H, wv.dk, wv.dv), dtype=torch.float32, device=dev),
                tape=torch.empty((wv.B, wv.T, wv.H, 3, wv.dk), dtype=torch.float32, device=dev),
                out=torch.empty((wv.B, wv.T, wv.H * wv.dv), dtype=torch.bfloat16, device=dev)))
        del st, cs
    torch.cuda.synchronize()

    def run(op, s):
        t = s.get("tok")
        if op in ("prefill", "prefill_softplus", "prefill_strong", "prefill_f32", "prefill_tiny"):
            lay = {"prefill_softplus": "layer_sp", "prefill_strong": "layer_st"}.get(op, "layer")
            abi.kda_prefill(s[lay], t["qkv"], t["f"], t["beta"], t["g_out"],
                            s["state"], s["conv"], s["out"], workspace=s["ws"], stream=stream)
        elif op == "varlen":
            abi.kda_prefill_varlen(s["layer"], var_cu, None, t["qkv"], t["f"], t["beta"], t["g_out"], s["state"],
                                   s["conv"], s["out"], workspace=s["ws"], stream=stream)
        elif op == "projection":
            abi.kda_input_projection(s["proj"], s["x"], s["qkv"], s["f"], s["beta"], s["g"], s["ws"], stream=stream)
        elif op in ("decode", "decode_softplus"):
            abi.kda_decode_step(s["layer" if op == "decode" else "layer_sp"], t["qkv"], t["f"], t["beta"],
                                t["g_out"], s["state"], s["conv"], s["out"], stream=stream)
        elif op == "verify":
            abi.kda_verify_block(s["layer"], t["qkv"], t["f"], t["beta"], t["g_out"], s["state"], s["conv"],
                                 s["snaps"], s["out"], stream=stream)
        elif op == "rollback":
            abi.kda_rollback(s["layer"], accepted, s["snaps"], t["qkv"], s["state"], s["conv"], stream=stream)
        elif op == "verify_tape":
            abi.kda_verify_block_tape(s["layer"], t["qkv"], t["f"], t["beta"], t["g_out"], s["state"], s["conv"],
                                      s["tape"], s["out"], stream=stream)
        elif op == "commit":
            abi.kda_commit_tape(s["layer"], accepted, s["tape"], t["qkv"], s["state"], s["conv"], stream=stream)

    seq = []
    for op in ops:
        seq.append(op)
        if op == "verify":
            seq += ["rollback", "verify_tape", "commit"]
        if op in ("prefill", "decode"):
            seq.append(op + "_softplus")
        if op == "prefill":
            seq += ["prefill_strong", "prefill_f32", "prefill_tiny"]

    def setof(op):
        if op.endswith("_softplus"):
            return op[: -len("_softplus")]
        if op == "prefill_strong":
            return "prefill"
        if op in ("prefill_f32", "prefill_tiny"):
            return op
        return "verify" if op in ("rollback", "verify_tape", "commit") else op

    for i in range(args.warmup):
        for op in seq:
            run(op, sets[setof(op)][i % nsets])
    torch.cuda.synchronize()

    K = args.steps
    # each call type runs K times back to back between one event pair, so the queue never drains
    ev = {op: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for op in seq}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for op in seq:
        e0, e1 = ev[op]
        e0.record(stream)
        for i in range(K):
            run(op, sets[setof(op)][i % nsets])
        e1.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    # the same K steps again with an event pair around every kernel (the library's timing hook),
    # for the per-kernel durations; kept out of the timed steps above so its events add no gaps
    abi.timing_enable(True)
    kernel_ms, op_kernel_ms = {}, {}
    for op in seq:
        for i in range(K):
            run(op, sets[setof(op)][i % nsets])
        torch.cuda.synchronize()
        for name, t in abi.timing_read():  # this call type's launches, in order
            kernel_ms.setdefault(name, []).append(t)
            op_kernel_ms.setdefault(op, {}).setdefault(name, []).append(t)
    abi.timing_enable(False)
    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    # each call on its own event pair, max(K, 50) calls per type: median and p10 / p90 per call
    KD = max(K, 50)
    dist = {}
    for op in seq:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(KD)]
        for i in range(KD):
            evs[i][0].record(stream)
            run(op, sets[setof(op)][i % nsets])
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in evs]
        dist[op] = {"ms_median": float(np.median(ts)), "ms_p10": float(np.percentile(ts, 10)),
                    "ms_p90": float(np.percentile(ts, 90)), "calls": KD}
    # cache-warm figure: the prefill on one buffer set, K calls back to back (inputs partly resident in
    # the 256 MB last-level cache), labelled as such and kept apart from the rotated-set numbers
    warm = None
    if "prefill" in ops:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        run("prefill", sets["prefill"][0])
        e0.record(stream)
        for i in range(K):
            run("prefill", sets["prefill"][0])
        e1.record(stream)
        torch.cuda.synchronize()
        warm = e0.elapsed_time(e1) / K
    ceil = hbm_ceilings(dev)
    ms_total = t_start.elapsed_time(t_end)
    mean = {op: ev[op][0].elapsed_time(ev[op][1]) / K for op in seq}

    res = {
        "metric": "KDA prefill tokens/s (H=32,128x128,T=4096) + decode state-update HBM GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_total / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_t4096 (B=1,T=4096,H=32,d=128,chunk 64) + the same tokens as 16 packed "
                               "sequences + their input projection (hidden 4096) + decode_b64 (B=64,H=32,d=128) "
                               "+ verify_b16 (B=16,T_d=8,H=32,d=128) with rollback and with the replay tape; "
                               "prefill_t4096 and decode_b64 again on the softplus decay branch; prefill_t4096 "
                               "with gate_lower_bound -8; the fp32 prefill at T=1024 and the small fp32 layer (T=64, H=2, "
                               "d=16)",
                   "io": "bf16 inputs and outputs, fp32 state and accumulation", "buffer_sets": nsets},
        "wall_s": wall,
    }
    detail = {}
    res["hbm_ceilings"] = {k: v["gbps"] for k, v in ceil.items()}
    res["hbm_ceilings"]["how"] = ("measured in this run, median of 5 each: a 1 GiB copy (1 GiB read + 1 GiB "
                                  "written) and a 1 GiB fill, by torch (copy_, fill_) and by the library's "
                                  "streaming copy (kda_measure_stream); copy and write are the higher of the "
                                  "two; read is torch sum over 1 GiB")
    copy_ceil = ceil["copy"]["gbps"]
    if "prefill" in ops:
        pb = prefill_bytes(1, wp.T, wp.H, wp.dk, wp.W)
        pf = prefill_alg_flops(wp.T, wp.H, wp.dk)
        res["value"] = wp.T / (mean["prefill"] * 1e-3)
        res["unit"] = "tokens/s"
        detail["prefill"] = {"ms_mean": mean["prefill"], "tokens_per_s": res["value"], "alg_bytes": pb,
                             "gbps": pb / (mean["prefill"] * 1e-3) / 1e9,
                             "hbm_frac": pb / (mean["prefill"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                             "alg_flops": pf, "alg_tflops": pf / (mean["prefill"] * 1e-3) / 1e12,
                             "cache_warm_ms": warm,
                             "cache_warm_note": "one buffer set, calls back to back: inputs partly in the last-level "
                                                "cache; not the headline (which rotates 4 sets)"}
    if "varlen" in ops:
        vb_ = sum(kernel_alg_bytes(k, wp, wd, wv, accepted) for k in
                  ("kda_chunk_prep_kernel[varlen]", "kda_chunk_state_kernel[varlen]", "kda_out_norm_kernel[varlen]"))
        detail["prefill_varlen"] = {"ms_mean": mean["varlen"], "tokens_per_s": wp.T / (mean["varlen"] * 1e-3),
                                    "alg_bytes": vb_, "gbps": vb_ / (mean["varlen"] * 1e-3) / 1e9,
                                    "sequences": VARLEN_SEQS, "lengths": var_lens}
        if "value" not in res:
            res["value"], res["unit"] = wp.T / (mean["varlen"] * 1e-3), "tokens/s"
    if "projection" in ops:
        fl = projection_flops(wj)
        tf = fl / (mean["projection"] * 1e-3) / 1e12
        detail["input_projection"] = {"ms_mean": mean["projection"], "flops": fl, "tflops": tf,
                                      "mfma_frac": tf / BF16_MFMA_PEAK_TFLOPS,
                                      "tokens_per_s": wj.T / (mean["projection"] * 1e-3),
                                      "workload": "T=4096, hidden=4096, H=32, d=128, rank 128, bf16 in and out"}
        if "value" not in res:
            res["value"], res["unit"] = wj.T / (mean["projection"] * 1e-3), "tokens/s"
    if "prefill" in ops:
        ms = mean["prefill_softplus"]
        detail["prefill_softplus"] = {"ms_mean": ms, "tokens_per_s": wp.T / (ms * 1e-3), "alg_bytes": pb,
                                      "gbps": pb / (ms * 1e-3) / 1e9,
                                      "workload": "prefill_t4096 with the softplus decay branch (no lower bound)"}
        ms = mean["prefill_strong"]
        detail["prefill_strong"] = {"ms_mean": ms, "tokens_per_s": wp.T / (ms * 1e-3), "alg_bytes": pb,
                                    "gbps": pb / (ms * 1e-3) / 1e9, "vs_prefill": ms / mean["prefill"],
                                    "workload": "prefill_t4096 with the bounded gate at gate_lower_bound = -8"}
        for op, wl, what in (("prefill_f32", wf, "fp32 io and out, B=1, T=1024, H=32, d=128, chunk 64 (the "
                                                 "vector-ALU prefill, internal chunk 32)"),
                             ("prefill_tiny", wt, "the small fp32 layer: B=1, T=64, H=2, d=16, chunk 16 "
                                                  "(launch-latency bound)")):
            ms = mean[op]
            nb = prefill_bytes(wl.B, wl.T, wl.H, wl.dk, wl.W, io_b=4, out_b=4)
            detail[op] = {"ms_mean": ms, "tokens_per_s": wl.B * wl.T / (ms * 1e-3), "alg_bytes": nb,
                          "gbps": nb / (ms * 1e-3) / 1e9, "workload": what}
    if "decode" in ops:
        db = decode_bytes(wd.B, wd.H, wd.dk, wd.W)
        gb = db / (mean["decode"] * 1e-3) / 1e9
        res["decode_state_update_gbps"] = gb
        detail["decode"] = {"ms_mean": mean["decode"], "alg_bytes": db, "gbps": gb,
                            "hbm_frac": gb / HBM_PEAK_GBPS}
        ms = mean["decode_softplus"]
        detail["decode_softplus"] = {"ms_mean": ms, "alg_bytes": db, "gbps": db / (ms * 1e-3) / 1e9,
                                     "hbm_frac": db / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                     "workload": "decode_b64 with the softplus decay branch"}
        if "value" not in res:
            res["value"], res["unit"] = gb, "GB/s"
    if "verify" in ops:
        vb = verify_bytes(wv.B, wv.T, wv.H, wv.dk, wv.W)
        rb = rollback_bytes(accepted, wv.H, wv.dk, wv.W)
        gv = vb / (mean["verify"] * 1e-3) / 1e9
        detail["verify"] = {"ms_mean": mean["verify"], "alg_bytes": vb, "gbps": gv,
                            "hbm_frac": gv / HBM_PEAK_GBPS}
        detail["rollback"] = {"ms_mean": mean["rollback"], "alg_bytes": rb,
                              "gbps": rb / (mean["rollback"] * 1e-3) / 1e9, "accepted": accepted}
        vtb = verify_tape_bytes(wv.B, wv.T, wv.H, wv.dk, wv.W)
        cb = commit_bytes(accepted, wv.H, wv.dk, wv.W)
        detail["verify_tape"] = {"ms_mean": mean["verify_tape"], "alg_bytes": vtb,
                                 "gbps": vtb / (mean["verify_tape"] * 1e-3) / 1e9}
        detail["commit_tape"] = {"ms_mean": mean["commit"], "alg_bytes": cb,
                                 "gbps": cb / (mean["commit"] * 1e-3) / 1e9}
        detail["speculative_block_ms"] = {"snapshots_verify_plus_rollback": mean["verify"] + mean["rollback"],
                                          "tape_verify_plus_commit": mean["verify_tape"] + mean["commit"]}
        if "value" not in res:
            res["value"], res["unit"] = gv, "GB/s"
    line_of = {"prefill": "prefill", "varlen": "prefill_varlen", "projection": "input_projection",
               "prefill_softplus": "prefill_softplus", "prefill_strong": "prefill_strong",
               "prefill_f32": "prefill_f32", "prefill_tiny": "prefill_tiny", "decode": "decode",
               "decode_softplus": "decode_softplus",
               "verify": "verify", "rollback": "rollback", "verify_tape": "verify_tape", "commit": "commit_tape"}
    for op, line in line_of.items():
        if op in op_kernel_ms and line in detail:
            # the call's kernels alone (their mean event time per launch), apart from host submission
            detail[line]["kernels_ms_mean"] = {n: float(np.mean(t)) for n, t in op_kernel_ms[op].items()}
        if op in dist and line in detail:
            detail[line].update(dist[op])
            if "alg_bytes" in detail[line] and detail[line]["alg_bytes"]:
                gm = detail[line]["alg_bytes"] / (dist[op]["ms_median"] * 1e-3) / 1e9
                detail[line]["gbps_median_call"] = gm
                detail[line]["frac_of_copy_ceiling"] = gm / copy_ceil
    # per kernel: average launch duration from the library's event pairs over the second pass
    kern = {}
    for name, ts in kernel_ms.items():
        avg = float(np.mean(ts))
        nb = kernel_alg_bytes(name, wp, wd, wv, accepted)
        kern[name] = {"ms_mean": avg, "ms_p10": float(np.percentile(ts, 10)), "ms_p90": float(np.percentile(ts, 90)),
                      "launches_per_step": len(ts) / K, "alg_bytes": nb,
                      "gbps": (nb / (avg * 1e-3) / 1e9) if nb else None}
        fl = kernel_alg_flops(name, wj)
        if fl:
            kern[name].update(flops=fl, tflops=fl / (avg * 1e-3) / 1e12,
                              mfma_frac=fl / (avg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS)
    detail["kernels"] = kern
    res["detail"] = detail
    # dominant kernel: the largest share of the step among the attention kernels of the headline
    # workloads (the variable-length and softplus lines run the same kernels on another table or
    # gate, and the input projection is a matrix-core GEMM line ahead of the layer: all are
    # reported beside them)
    share = lambda n: kern[n]["ms_mean"] * kern[n]["launches_per_step"]
    hbm = [n for n in kern if "[varlen]" not in n and "[softplus]" not in n and "[strong]" not in n
           and kern[n]["alg_bytes"]]
    if not hbm:  # a run of one side line (--only varlen): its own kernels
        hbm = [n for n in kern if kern[n]["alg_bytes"]]
    if hbm:
        name = max(hbm, key=share)
        k = kern[name]
        achieved = k["gbps"]
        tr = stored_traffic(name)
        res["roofline"] = {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": tr,
                           "traffic_source": ("profiles/pmc_traffic.json: rocprofv3 FETCH_SIZE and WRITE_SIZE runs "
                                              "on these sources, scaled by a plain copy of known size; not measured "
                                              "in this run") if tr is not None else None,
                           "frac_of_measured_copy_ceiling": achieved / copy_ceil,
                           "alg_bytes_per_launch": k["alg_bytes"], "ms_per_launch": k["ms_mean"]}
        if "prefill" in detail:
            pl = detail["prefill"]
            res["roofline"]["prefill_mfma"] = {
                "alg_tflops": pl["alg_tflops"], "peak": BF16_MFMA_PEAK_TFLOPS,
                "frac": pl["alg_tflops"] / BF16_MFMA_PEAK_TFLOPS,
                "issued_frac_by_kernel": {kn: stored_mfma_issued(kn) for kn in
                                          ("kda_chunk_prep_kernel", "kda_chunk_state_kernel")},
                "note": "algorithmic dense-tile flops of the prefill call over its mean call time; issued fraction "
                        "from profiles/pmc_mfma.json (SQ_INSTS_MFMA x 16,384 flop over the dispatch time, of the "
                        "2.5 PFLOP/s dense bf16 peak), null when those counters were taken on other sources"}
    else:  # --only projection: its GEMM against the dense bf16 matrix-core peak
        name = max((n for n in kern if kern[n].get("flops")), key=share)
        k = kern[name]
        res["roofline"] = {"kernel": name, "bound": "mfma", "achieved": k["tflops"], "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": k["mfma_frac"], "traffic": None,
                           "alg_flops_per_launch": k["flops"], "ms_per_launch": k["ms_mean"]}
    if not args.no_cpu_baseline and "prefill" in ops:
        log("timing the oracle on the host ...")
        res["cpu_baseline"] = cpu_baseline(args.cpu_heads, wp.T)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
