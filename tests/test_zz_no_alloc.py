"""fd_paged_decode_noalloc: the paged decode on the library's static per-GPU scratch.

Called through the C ABI and compared with fd_paged_decode on its own workspace
(same plan, same kernels: the same bits) and with the float64 oracle (|gpu - ref|
<= 2e-3 + 1e-2 |ref| for 16-bit inputs), on two calls in a row, the second one
smaller, so the second reads a scratch that still holds the first call's partials.
"""
import ctypes
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
    sys.__stderr__.write(f"[gpu-case] noalloc {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def noalloc(g, d, opt=None, total_kv=None):
    """One call of fd_paged_decode_noalloc through the C ABI."""
    o = torch.empty_like(g["q"])
    B, H, D = g["q"].shape
    num_pages, ps, Hkv, _ = g["k_cache"].shape
    rc = fd.lib().fd_paged_decode_noalloc(
        g["q"].data_ptr(), g["k_cache"].data_ptr(), g["v_cache"].data_ptr(), g["block_table"].data_ptr(),
        g["seq_lens"].data_ptr(), ps, o.data_ptr(), d["scale"], B, H, Hkv, D, num_pages, g["block_table"].shape[1],
        d["max_seq_len"], d["total_kv"] if total_kv is None else total_kv, fd.binding.FD_DTYPE[g["q"].dtype],
        ctypes.byref(opt) if opt is not None else None, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, fd.lib().fd_last_error().decode()
    return o


def with_workspace(g, d, opt=None, total_kv=None):
    return fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"],
                              scale=d["scale"], max_seq_len=d["max_seq_len"],
                              total_kv=d["total_kv"] if total_kv is None else total_kv, opt=opt)


def check(o, d):
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           d["page_size"], d["scale"])
    got = o.cpu().to(torch.float64).numpy()
    err = np.abs(got - ref)
    assert (err <= ATOL + RTOL * np.abs(ref)).all(), f"max|err| {err.max():.3e}"


def test_noalloc_two_calls_match_paged_decode(device):
    big = inputs.paged_inputs(16, 32, 8, 128, "bf16", 16,
                              np.random.default_rng(61).integers(1, 6000, 16).tolist(), 62)
    small = inputs.paged_inputs(3, 32, 8, 128, "bf16", 16, [5, 700, 2100], 63)
    for name, d in (("16 sequences", big), ("3 sequences", small)):
        g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        plan = fd.paged_plan(d["B"], 32, 8, "bf16", 16, d["max_seq_len"], d["total_kv"])
        assert plan["merge"] != 0 and plan["workspace_bytes"] <= fd.binding.NOALLOC_SCRATCH_BYTES
        announce(f"{name}: plan chunk {plan['chunk']} splits {plan['num_splits']} work_list {plan['work_list']}")
        o = noalloc(g, d)
        ref = with_workspace(g, d)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), name
        check(o, d)


def test_noalloc_persistent_launch_uses_the_scratch_counters(device):
    """The persistent launch claims its items through two counters in the block at the
    head of the static scratch, which its last workgroup returns to zero: two calls in
    a row (the second smaller) give the bits of the same plan on a workspace."""
    for lens, seed in (([300, 4000, 2049, 64, 3333, 0, 17], 64), ([700, 1500], 65)):
        d = inputs.paged_inputs(len(lens), 32, 8, 128, "bf16", 16, lens, seed)
        g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
        opt = fd.options(force_chunk=256, launch="persistent")
        plan = fd.paged_plan(d["B"], 32, 8, "bf16", 16, d["max_seq_len"], d["total_kv"], 0, opt)
        assert plan["persistent"] == 1
        announce(f"persistent, {len(lens)} sequences, work list {plan['work_list']}")
        o = noalloc(g, d, opt=opt)
        ref = with_workspace(g, d, opt=opt)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)
        check(o, d)


def test_noalloc_refuses_plans_beyond_the_scratch(device):
    """A plan whose partials exceed the static scratch is refused before anything is
    launched (nothing is read from the small stand-in buffers)."""
    B, H, Hkv = 512, 64, 8
    plan = fd.paged_plan(B, H, Hkv, "bf16", 16, 65536, 0)
    assert plan["workspace_bytes"] > fd.binding.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(4096, dtype=torch.int32, device=device)
    x = torch.zeros(4096, dtype=torch.bfloat16, device=device)
    announce("refusal")
    rc = fd.lib().fd_paged_decode_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), t.data_ptr(), t.data_ptr(), 16,
                                          x.data_ptr(), 0.1, B, H, Hkv, 128, 4096, 4096, 65536, 0, 2, None,
                                          torch.cuda.current_stream().cuda_stream)
    assert fd.lib().fd_status_string(rc).decode() == "FD_ERR_WORKSPACE"
    assert "static scratch" in fd.lib().fd_last_error().decode()
