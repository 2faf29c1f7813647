"""The library's streaming copy (kda_measure_stream), which bench.py uses for its HBM ceilings:
a copy must reproduce its source bit for bit and a fill must write zeros, over a size whose
16-byte words do not divide evenly into the kernel's unrolled grid strides."""
import pytest
import torch

from hybrid_linear_attention_kda_amd import abi


@pytest.mark.gpu
def test_measure_stream_copies_and_fills():
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    n = (1 << 22) + 12  # int32 words: 16 MiB + 48 bytes
    x = torch.randint(-(1 << 31), (1 << 31) - 1, (n,), generator=g, dtype=torch.int32).to(dev)
    y = torch.full_like(x, 5)
    abi.measure_stream(y, x)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
    abi.measure_stream(y)
    torch.cuda.synchronize()
    assert int((y != 0).sum()) == 0
    assert abi.load().kda_measure_stream(None, None, 16, None) == abi.KDA_ERR_INVALID_ARGUMENT
