"""GPU parity of fd_prefill (many-query attention, optional causal mask) against
the float64 oracle, through the C ABI. Tolerance as for the decode path with
16-bit inputs: |gpu - ref| <= 2e-3 + 1e-2 |ref| against the unrounded oracle."""
import sys

import numpy as np
import pytest
import torch

import decode_attention_13_amd as fd
import oracle
from decode_attention_13_amd import inputs

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] prefill {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def run(d, dev, causal):
    o = fd.fd_prefill(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), scale=d["scale"], causal=causal)
    torch.cuda.synchronize()
    return o.cpu()


def assert_close(got, ref, what):
    got = got.to(torch.float64).numpy()
    err = np.abs(got - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    assert not bad.any(), f"{what}: max|err| {err.max():.3e}, {int(bad.sum())}/{bad.size} outside tolerance"


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_pages_harness_shape(dtype, causal, device):
    """The FA page's harness: 8 heads, N = 1000 (not a multiple of any block), causal and
    not; head dim 128 here."""
    d = inputs.prefill_inputs(1, 1000, 8, 8, 128, dtype, 500)
    announce(f"harness {dtype} causal={causal}")
    o = run(d, device, causal)
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
    assert_close(o, ref, f"N=1000 {dtype} causal={causal}")


@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 63, 64, 65, 127, 129, 200])
def test_lengths(N, device):
    """Every tail shape of the 64-query and 32-key tiles, GQA 8/2, two sequences."""
    d = inputs.prefill_inputs(2, N, 8, 2, 128, "bf16", 510 + N)
    for causal in (True, False):
        announce(f"N={N} causal={causal}")
        o = run(d, device, causal)
        ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
        assert_close(o, ref, f"N={N} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_first_row_is_exact(dtype, device):
    """Causal row 0 sees one key: o = v_0 of its KV head, bit for bit."""
    d = inputs.prefill_inputs(2, 130, 6, 3, 128, dtype, 520)
    announce(f"first row {dtype}")
    o = run(d, device, True)
    want = d["v"][:, 0].repeat_interleave(2, dim=1)
    assert torch.equal(o[:, 0], want)


def test_workload_prefill_bf16_h32_n4096_causal(device):
    """Full size (the benchmark's launch); three heads against the oracle, every
    output finite."""
    w = inputs.PREFILL_WORKLOADS["prefill_bf16_h32_n4096_causal"]
    d = w.make()
    announce(w.name)
    o = run(d, device, True)
    assert torch.isfinite(o.float()).all()
    heads = [0, 17, 31]
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], True, heads=heads)
    assert_close(o[:, :, heads], ref, w.name)


def test_workload_gqa(device):
    w = inputs.PREFILL_WORKLOADS["prefill_f16_b2_h32_kv8_n2048_causal"]
    d = w.make()
    announce(w.name)
    o = run(d, device, True)
    heads = [3, 12, 30]
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], True, heads=heads)
    assert_close(o[:, :, heads], ref, w.name)
