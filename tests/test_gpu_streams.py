"""Calls on a stream other than the current one, through the binding.

The binding allocates the output and (when none is passed) the workspace on the
current stream, zero-filling a decode workspace there; the library then runs on
the caller's stream. That stream must first wait for the fill, and the memory
must not return to the allocator before the stream's work is done. Each test
runs the same call on the current stream and on a side stream (a torch stream
object and a raw handle) while the current stream is kept busy, and compares
the results bit for bit."""
import sys

import pytest
import torch

import decode_attention_13_amd as fd
from decode_attention_13_amd import inputs

pytestmark = pytest.mark.gpu


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] streams {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def _busy(device):
    """Queue some work on the current stream, so a side stream that does not wait
    for it would run ahead."""
    x = torch.randn(2048, 2048, device=device)
    for _ in range(4):
        x = x @ x
        x = x / x.abs().amax()
    return x


@pytest.mark.parametrize("handle", ["stream", "raw"])
def test_decode_on_a_side_stream(handle, device):
    d = inputs.single_inputs(32, 8, 4096, 128, "bf16", 700)
    q, k, v = d["q"].to(device), d["k"].to(device), d["v"].to(device)
    want = fd.fd_decode(q, k, v, scale=d["scale"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    announce(f"decode on a side stream ({handle})")
    outs = []
    for _ in range(3):
        _busy(device)
        outs.append(fd.fd_decode(q, k, v, scale=d["scale"], stream=side if handle == "stream" else side.cuda_stream))
    torch.cuda.synchronize()
    for got in outs:
        assert torch.equal(got, want)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_on_a_side_stream(dtype, device):
    d = inputs.prefill_inputs(2, 300, 8, 2, 128, dtype, 701)
    q, k, v = d["q"].to(device), d["k"].to(device), d["v"].to(device)
    want = fd.fd_prefill(q, k, v, scale=d["scale"], causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    announce(f"prefill {dtype} on a side stream")
    outs = []
    for _ in range(3):
        _busy(device)
        outs.append(fd.fd_prefill(q, k, v, scale=d["scale"], causal=True, stream=side))
    torch.cuda.synchronize()
    for got in outs:
        assert torch.equal(got, want)
