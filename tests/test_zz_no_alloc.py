"""The workspace-free prefill entry point against kda_prefill with a caller workspace.

kda_prefill_noalloc runs the same kernels with the library's fixed scratch array as the workspace;
two calls in a row (the second smaller, so it reuses the array the first left behind) must match
kda_prefill to the bf16 bar, and bit for bit (same kernels, same inputs).
"""
import numpy as np
import pytest
import torch

from hybrid_linear_attention_kda_amd import abi
from hybrid_linear_attention_kda_amd import inputs as I
from hybrid_linear_attention_kda_amd import tensors as TT
from parity_util import TOL, rel_err, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(wl, inp, S0, C0, noalloc):
    layer = TT.make_layer(wl, inp, DEV)
    tok = TT.token_tensors(wl, inp, 0, wl.T, DEV)
    st = torch.from_numpy(S0).to(DEV)
    cs = TT.to_device(C0, wl.io, DEV)
    out = torch.empty((wl.B, wl.T, wl.H * wl.dv), dtype=torch.float32, device=DEV)
    if noalloc:
        abi.kda_prefill_noalloc(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out)
    else:
        ws = torch.empty(abi.kda_prefill_workspace_size(layer, wl.B, wl.T), dtype=torch.uint8, device=DEV)
        abi.kda_prefill(layer, tok["qkv"], tok["f"], tok["beta"], tok["g_out"], st, cs, out, workspace=ws)
    torch.cuda.synchronize()
    return out, st, cs


def test_noalloc_prefill_matches_workspace_prefill_twice():
    cases = [I.WORKLOADS["prefill_t4096"].with_(T=1472, seed=80),          # the largest call the scratch holds
             I.WORKLOADS["prefill_t4096"].with_(T=130, H=4, B=3, seed=81)]  # then a smaller one
    for wl in cases:
        say(f"case kda_prefill_noalloc B={wl.B} T={wl.T} H={wl.H} vs kda_prefill with a workspace")
        inp = I.generate(wl)
        rng = np.random.default_rng(wl.seed)
        S0 = (rng.standard_normal(inp["state0"].shape) * 0.3).astype(np.float32)
        C0 = I.round_to_io(rng.standard_normal(inp["conv_state0"].shape), "bf16")
        o1, s1, c1 = _run(wl, inp, S0, C0, noalloc=True)
        o2, s2, c2 = _run(wl, inp, S0, C0, noalloc=False)
        for name, a, b in (("out", o1, o2), ("state", s1, s2), ("conv_state", c1, c2)):
            e = rel_err(TT.to_host_f64(a), TT.to_host_f64(b))
            say(f"  {name}: rel err {e:.3e}, bit-identical {torch.equal(a, b)}")
            assert e <= TOL["bf16"]
            assert torch.equal(a, b), name
