"""GPU parity of fd_prefill (many-query attention, optional causal mask) against
the float64 oracle, through the C ABI. Tolerance as for the decode path with
16-bit inputs: |gpu - ref| <= 2e-3 + 1e-2 |ref| against the unrounded oracle.

bf16 calls go through the binding's default, the workspace path (V converted to
f16, P.V on f16 MFMAs, sequences whose V does not convert rerun with the split
P); the tests marked "split" pass no workspace and run the split-P kernel alone."""
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


def run(d, dev, causal, ws=None):
    o = fd.fd_prefill(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), scale=d["scale"], causal=causal, ws=ws)
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
    """Causal row 0 sees one key: o = v_0 of its KV head, bit for bit (bf16 V
    goes through f16, exact for 2^-17 <= |v| < 65536; the seeded row has no
    smaller nonzero magnitude)."""
    d = inputs.prefill_inputs(2, 130, 6, 3, 128, dtype, 520)
    v0 = d["v"][:, 0].to(torch.float32).abs()
    assert not ((v0 > 0) & (v0 < 2.0 ** -17)).any()
    announce(f"first row {dtype}")
    o = run(d, device, True)
    want = d["v"][:, 0].repeat_interleave(2, dim=1)
    assert torch.equal(o[:, 0], want)


@pytest.mark.parametrize("path", ["workspace", "split"])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_tiles_beyond_f16(causal, path, device):
    """bf16 V far outside f16's range (|v| from 65280 up to 1e30) in key rows of
    several tiles, loaded by different waves: P.V on bf16 MFMAs with P split in
    a truncated hi and a rounded lo part keeps them exact to 16 bits of P. With
    the workspace both sequences are flagged and take that kernel too.

    Outputs here can be small sums of terms near 1e4 that cancel, so the bound
    also carries the conditioning of each output: P is kept to a relative 2^-15
    (hi + lo), which moves o[d] by at most 2^-15 * sum_k w_k |v_k[d]|; the test
    allows 2^-12 of it (the oracle's output for |V|)."""
    d = inputs.prefill_inputs(2, 200, 8, 2, 128, "bf16", 530)
    v = d["v"].to(torch.float32)
    for key, mult in [(32 + 3, 3e5), (64 + 21, -7e4), (160 + 30, 1e30), (160 + 9, 2e5)]:
        v[:, key] *= mult
    v[0, 96 + 12, 1, 5] = 65280.0
    v[1, 192 + 4, 0, 77] = -65536.0
    d["v"] = v.to(torch.bfloat16)
    assert d["v"][0, 96 + 12, 1, 5].item() == 65280.0
    announce(f"bf16 tiles beyond f16, causal={causal}, {path}")
    ws = None
    if path == "workspace":
        ws = torch.empty(fd.prefill_workspace_size(2, 200, 2, torch.bfloat16), dtype=torch.uint8, device=device)
    o = run(d, device, causal, ws if path == "workspace" else False)
    if path == "workspace":
        flags = fd.prefill_flags(ws, 2, 200, 2).cpu()
        assert flags[:, :4].amax(dim=1).tolist() == [1, 1]  # 400 rows: 4 chunks of 128 per sequence
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
    cond, _ = oracle.prefill_attention(d["q"], d["k"], d["v"].abs(), d["scale"], causal)
    err = np.abs(o.to(torch.float64).numpy() - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref) + 2.0 ** -12 * cond)
    assert not bad.any(), f"wide V causal={causal}: {int(bad.sum())} outside, max|err| {err.max():.3e}"


@pytest.mark.parametrize("causal", [True, False])
def test_long_prompt_sampled_rows(causal, device):
    """N = 32768, one sequence, 4 query heads on 2 KV heads, bf16: a query tile
    walks up to 1024 key tiles, so the LDS rings wrap hundreds of times. Sampled
    rows (tile edges, the last rows, random ones) against the float64 oracle's
    decode of that row's query: over keys 0..i with the causal mask, else over
    all N keys (a prefill row is the decode of its query)."""
    N, H, Hkv = 32768, 4, 2
    d = inputs.prefill_inputs(1, N, H, Hkv, 128, "bf16", 560)
    announce(f"long prompt N={N} causal={causal}")
    o = run(d, device, causal)
    rng = np.random.default_rng(561)
    rows = sorted(set([0, 1, 31, 32, 127, 128, 129, N // 2, N - 2, N - 1] + rng.integers(0, N, 14).tolist()))
    for i in rows:
        keys = i + 1 if causal else N
        ref, _ = oracle.decode_attention(d["q"][0, i], d["k"][0, :keys], d["v"][0, :keys], d["scale"])
        assert_close(o[0, i], ref, f"N={N} causal={causal} row {i}")


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


@pytest.mark.parametrize("scale", [-0.0883883, 0.0, 0.5, 3.0])
@pytest.mark.parametrize("causal", [True, False])
def test_scales(scale, causal, device):
    """A negative scale (its sign goes into Q on the device), a zero scale (every
    visible key weighs the same), and large scales whose scores spread over many
    powers of two, so the running max moves by more than the lazy threshold."""
    d = inputs.prefill_inputs(1, 300, 4, 2, 128, "bf16", 530)
    announce(f"scale={scale} causal={causal}")
    o = fd.fd_prefill(d["q"].to(device), d["k"].to(device), d["v"].to(device), scale=scale, causal=causal)
    torch.cuda.synchronize()
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], scale, causal)
    assert_close(o.cpu(), ref, f"scale={scale} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rising_scores_rescale_every_tile(dtype, device):
    """Keys built so that every query's best score grows by about 12 (log2 units)
    from one 32-key tile to the next: the running max moves on every tile and the
    accumulators are rescaled each time."""
    N, D = 256, 128
    g = torch.Generator().manual_seed(540)
    q = torch.randn(1, N, 2, D, generator=g) * 0.1
    q[..., 0] = 1.0
    k = torch.randn(1, N, 1, D, generator=g) * 0.1
    k[..., 0] = (torch.arange(N) // 32).to(torch.float32)[None, :, None] * 8.0 / (1.4427 * 0.75)
    v = torch.randn(1, N, 1, D, generator=g)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    q, k, v = q.to(tdt), k.to(tdt), v.to(tdt)
    scale = 1.1
    announce(f"rising scores {dtype}")
    for causal in (True, False):
        o = fd.fd_prefill(q.to(device), k.to(device), v.to(device), scale=scale, causal=causal)
        torch.cuda.synchronize()
        ref, _ = oracle.prefill_attention(q, k, v, scale, causal)
        assert_close(o.cpu(), ref, f"rising {dtype} causal={causal}")


@pytest.mark.parametrize("B,N,H,Hkv", [(1, 300, 6, 1), (3, 257, 12, 3), (2, 190, 16, 2), (1, 96, 1, 1)])
def test_head_groupings(B, N, H, Hkv, device):
    """MQA (one KV head), GQA 4 and 8, and a single head; (sequence, head) unit
    counts that are and are not multiples of the XCD count, so both workgroup
    orders of the grid run."""
    d = inputs.prefill_inputs(B, N, H, Hkv, 128, "bf16", 550 + H)
    for causal in (True, False):
        announce(f"B={B} N={N} H={H}/{Hkv} causal={causal}")
        o = run(d, device, causal)
        ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
        assert_close(o, ref, f"B={B} N={N} H={H}/{Hkv} causal={causal}")


def _chunks(N, Hkv):
    rows = N * Hkv
    per = max(128, -(-rows // 1024))
    return -(-rows // per)


def test_bf16_workspace_flags_per_sequence(device):
    """Three sequences, one V value of 70000 in sequence 1 (no f16 for it) and
    65280, the largest bf16 value below 65536, in sequence 2 (exact in f16):
    only sequence 1 is flagged and rerun with the split P; all three match the
    oracle. The same workspace then serves a batch with no such value, and no
    flag of the first call survives."""
    B, N, H, Hkv = 3, 300, 8, 2
    d = inputs.prefill_inputs(B, N, H, Hkv, 128, "bf16", 570)
    v = d["v"].clone()
    v[1, 217, 1, 40] = 70000.0
    v[2, 5, 0, 3] = -65280.0
    assert v[1, 217, 1, 40].item() == 70144.0 and v[2, 5, 0, 3].item() == -65280.0  # bf16 rounding
    d["v"] = v
    ws = torch.empty(fd.prefill_workspace_size(B, N, Hkv, torch.bfloat16), dtype=torch.uint8, device=device)
    c = _chunks(N, Hkv)
    for causal in (True, False):
        announce(f"flags per sequence causal={causal}")
        o = run(d, device, causal, ws)
        flags = fd.prefill_flags(ws, B, N, Hkv)[:, :c].cpu()
        assert flags.amax(dim=1).tolist() == [0, 1, 0]
        assert flags[1].tolist() == [1 if i == (217 * Hkv + 1) // 128 else 0 for i in range(c)]
        ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
        assert_close(o, ref, f"flags per sequence causal={causal}")
    d2 = inputs.prefill_inputs(B, N, H, Hkv, 128, "bf16", 571)
    announce("flags cleared by the next call")
    o = run(d2, device, True, ws)
    assert int(fd.prefill_flags(ws, B, N, Hkv)[:, :c].max()) == 0
    ref, _ = oracle.prefill_attention(d2["q"], d2["k"], d2["v"], d2["scale"], True)
    assert_close(o, ref, "second call")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("N", [1, 33, 1000])
def test_bf16_split_path(N, causal, device):
    """bf16 without a workspace: the split-P kernel alone, GQA 8/2, two sequences."""
    d = inputs.prefill_inputs(2, N, 8, 2, 128, "bf16", 580 + N)
    announce(f"split path N={N} causal={causal}")
    o = run(d, device, causal, False)
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], causal)
    assert_close(o, ref, f"split N={N} causal={causal}")


def test_bf16_large_batch_many_chunks(device):
    """A sequence whose V rows exceed 1024 * 128 (N = 8192, Hkv = 32): chunks of
    more than 128 rows, the flag row full; one value of 1e5 near the end of the
    second sequence flags it alone. Sampled rows against the oracle's decode."""
    B, N, H, Hkv = 2, 8192, 32, 32
    d = inputs.prefill_inputs(B, N, H, Hkv, 128, "bf16", 590)
    v = d["v"].clone()
    v[1, N - 3, 30, 100] = 1e5
    d["v"] = v
    c = _chunks(N, Hkv)
    assert c == 1024
    ws = torch.empty(fd.prefill_workspace_size(B, N, Hkv, torch.bfloat16), dtype=torch.uint8, device=device)
    announce("large batch, full flag rows")
    o = run(d, device, True, ws)
    flags = fd.prefill_flags(ws, B, N, Hkv).cpu()
    assert flags[0].max().item() == 0 and flags[1].tolist() == [1 if i == c - 1 else 0 for i in range(c)]
    for b, i, h in [(0, 0, 0), (0, N - 1, 31), (1, 4000, 17), (1, N - 1, 30), (1, N - 2, 31)]:
        g = h // (H // Hkv)
        ref, _ = oracle.decode_attention(d["q"][b, i, h:h + 1], d["k"][b, :i + 1, g:g + 1], d["v"][b, :i + 1, g:g + 1],
                                         d["scale"])
        assert_close(o[b, i, h:h + 1], ref, f"large batch b={b} row {i} head {h}")


@pytest.mark.parametrize("case", range(12))
def test_seeded_random_shapes(case, device):
    """Twelve seeded draws of (B, N, H, Hkv, dtype, causal, scale): ragged N, GQA
    from 1 to 8, both dtypes, both masks; bf16 through the workspace path, and
    in cases 2, 6 and 10 also without it. Every output against the oracle."""
    rng = np.random.default_rng(900 + case)
    Hkv = int(rng.choice([1, 2, 4]))
    H = Hkv * int(rng.choice([1, 2, 3, 8]))
    B = int(rng.integers(1, 4))
    N = int(rng.integers(1, 420))
    dtype = ["bf16", "f16"][case % 2]
    causal = bool(rng.integers(0, 2))
    d = inputs.prefill_inputs(B, N, H, Hkv, 128, dtype, 910 + case)
    scale = float(rng.choice([d["scale"], 0.3, -0.05]))
    paths = [None, False] if dtype == "bf16" and case % 4 == 2 else [None]
    ref, _ = oracle.prefill_attention(d["q"], d["k"], d["v"], scale, causal)
    for ws in paths:
        announce(f"seeded case {case}: B={B} N={N} H={H}/{Hkv} {dtype} causal={causal} scale={scale:.3f} ws={ws}")
        o = fd.fd_prefill(d["q"].to(device), d["k"].to(device), d["v"].to(device), scale=scale, causal=causal, ws=ws)
        torch.cuda.synchronize()
        assert_close(o.cpu(), ref, f"case {case}")
