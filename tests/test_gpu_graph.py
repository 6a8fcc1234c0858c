"""Decode steps captured in a HIP graph (torch.cuda.graph) and replayed.

A serving loop captures its decode step once and replays it; the library's
default path is plain kernel launches on the caller's stream (no allocation,
no host synchronisation, no memset), so it can be captured. Each test captures
a step with pre-allocated inputs, output and workspace, then replays it several
times with new inputs copied into the captured buffers, eager work and
synchronisations between the replays, and checks every replay bit for bit
against an eager call of the same plan on the same inputs (and once against the
float64 oracle, |gpu - ref| <= 2e-3 + 1e-2 |ref|). The persistent launch's
counters and the fused merge's counters are left at zero by every replay.
"""
import sys

import numpy as np
import pytest
import torch

import decode_attention_13_amd as fd
import oracle
from decode_attention_13_amd import inputs

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-3, 1e-2
REPLAYS = 4


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] graph {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def close_to(o, ref):
    err = np.abs(o.cpu().to(torch.float64).numpy() - ref)
    return bool((err <= ATOL + RTOL * np.abs(ref)).all())


@pytest.mark.parametrize("merge", ["kernel", "fused"])
def test_contiguous_decode_step_replays(merge, device):
    """The 4k-token 32-head bf16 decode (split kernel + merge kernel, or one fused
    launch) captured once and replayed with four different queries."""
    H, Hkv, S = 32, 32, 4096
    d = inputs.single_inputs(H, Hkv, S, 128, "bf16", 501)
    qs = [inputs.single_inputs(H, Hkv, S, 128, "bf16", 502 + r)["q"].to(device) for r in range(REPLAYS)]
    k, v = d["k"].to(device), d["v"].to(device)
    opt = fd.options(merge=merge)
    plan = fd.decode_plan(H, Hkv, S, "bf16", 0, opt)
    assert plan["merge"] == {"kernel": 1, "fused": 2}[merge]
    q_static = qs[0].clone()
    o_static = torch.empty_like(q_static)
    ws = fd.new_workspace(plan["workspace_bytes"], device)
    ws_eager = fd.new_workspace(plan["workspace_bytes"], device)
    torch.cuda.synchronize()
    announce(f"contiguous capture, merge {merge}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_decode(q_static, k, v, o=o_static, scale=d["scale"], ws=ws, opt=opt)
    for r in range(REPLAYS):
        announce(f"contiguous replay {r}")
        q_static.copy_(qs[r])
        g.replay()
        torch.cuda.synchronize()
        got = o_static.clone()
        ref = fd.fd_decode(qs[r], k, v, scale=d["scale"], ws=ws_eager, opt=opt)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        assert torch.all(ws[:fd.binding.WS_COUNTER_BYTES] == 0), r
        if r == REPLAYS - 1:
            want, _ = oracle.decode_attention(qs[r].cpu(), d["k"], d["v"], d["scale"])
            assert close_to(got, want)


def _paged_case(device):
    lens = np.random.default_rng(511).integers(0, 5000, 24).tolist()
    d = inputs.paged_inputs(len(lens), 32, 8, 128, "bf16", 16, lens, 512)
    qs = [inputs.paged_inputs(len(lens), 32, 8, 128, "bf16", 16, lens, 513 + r)["q"].to(device)
          for r in range(REPLAYS)]
    g = {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    return lens, d, g, qs


def test_paged_persistent_step_replays(device):
    """A ragged 24-sequence GQA4 batch on the persistent launch (claim counters in
    the workspace) captured once and replayed with four different queries."""
    lens, d, g, qs = _paged_case(device)
    opt = fd.options(force_chunk=256, launch="persistent")
    plan = fd.paged_plan(len(lens), 32, 8, "bf16", 16, max(lens), sum(lens), 0, opt)
    assert plan["persistent"] == 1
    q_static = qs[0].clone()
    o_static = torch.empty_like(q_static)
    ws = fd.new_workspace(plan["workspace_bytes"], device)
    ws_eager = fd.new_workspace(plan["workspace_bytes"], device)

    def step(q, o, w):
        return fd.fd_paged_decode(q, g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16, o=o,
                                  scale=d["scale"], max_seq_len=max(lens), total_kv=sum(lens), opt=opt, ws=w)

    torch.cuda.synchronize()
    announce("paged capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q_static, o_static, ws)
    for r in range(REPLAYS):
        announce(f"paged replay {r}")
        q_static.copy_(qs[r])
        graph.replay()
        torch.cuda.synchronize()
        got = o_static.clone()
        ref = step(qs[r], None, ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        assert torch.all(ws[:fd.binding.WS_COUNTER_BYTES] == 0), r
        if r == REPLAYS - 1:
            want, _ = oracle.paged_decode_attention(qs[r].cpu(), d["k_cache"], d["v_cache"], d["block_table"],
                                                    d["seq_lens"], 16, d["scale"])
            assert close_to(got, want)


def test_paged_noalloc_step_replays(device):
    """fd_paged_decode_noalloc, for callers that cannot allocate, captured once
    (after a first eager call has set up the static scratch) and replayed."""
    lens, d, g, qs = _paged_case(device)
    opt = fd.options(force_chunk=256, launch="persistent")
    q_static = qs[0].clone()
    o_static = torch.empty_like(q_static)

    def step(q, o):
        return fd.fd_paged_decode_noalloc(q, g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                          o=o, scale=d["scale"], max_seq_len=max(lens), total_kv=sum(lens),
                                          opt=opt)

    announce("noalloc first eager call")
    first = step(qs[0], None).clone()
    torch.cuda.synchronize()
    announce("noalloc capture")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q_static, o_static)
    for r in range(REPLAYS):
        announce(f"noalloc replay {r}")
        q_static.copy_(qs[r])
        graph.replay()
        torch.cuda.synchronize()
        got = o_static.clone()
        ref = step(qs[r], None)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        if r == 0:
            assert torch.equal(got, first)


def test_bf16_prefill_workspace_replays(device):
    """The bf16 prefill with a workspace (conversion, attention, split-P rerun:
    three launches, no memset) captured once and replayed with new q, k and v
    copied in; the second set holds a value no f16 can carry, so one replay
    takes the split-P kernel for that sequence. Every replay equals an eager
    call bit for bit."""
    B, N, H, Hkv = 2, 300, 8, 2
    sets = [inputs.prefill_inputs(B, N, H, Hkv, 128, "bf16", 600 + r) for r in range(3)]
    sets[1]["v"][1, 150, 0, 9] = 1e6
    dev = [{n: sets[r][n].to(device) for n in ("q", "k", "v")} for r in range(3)]
    static = {n: dev[0][n].clone() for n in ("q", "k", "v")}
    o_static = torch.empty_like(static["q"])
    need = fd.prefill_workspace_size(B, N, Hkv, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    ws_eager = torch.empty(need, dtype=torch.uint8, device=device)
    scale = sets[0]["scale"]
    fd.fd_prefill(static["q"], static["k"], static["v"], o=o_static, scale=scale, causal=True, ws=ws)
    torch.cuda.synchronize()
    announce("prefill capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fd.fd_prefill(static["q"], static["k"], static["v"], o=o_static, scale=scale, causal=True, ws=ws)
    for r in range(REPLAYS):
        announce(f"prefill replay {r}")
        for n in ("q", "k", "v"):
            static[n].copy_(dev[r % 3][n])
        g.replay()
        torch.cuda.synchronize()
        got = o_static.clone()
        ref = fd.fd_prefill(dev[r % 3]["q"], dev[r % 3]["k"], dev[r % 3]["v"], scale=scale, causal=True, ws=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), r
        flagged = fd.prefill_flags(ws, B, N, Hkv)[:, :5].amax(dim=1).tolist()
        assert flagged == ([0, 1] if r % 3 == 1 else [0, 0]), (r, flagged)
