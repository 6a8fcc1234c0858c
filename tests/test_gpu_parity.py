"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerance (elementwise, the allclose convention): |gpu - ref| <= atol + rtol*|ref|
with the unrounded float64 oracle as ref; bf16/f16 inputs: atol 2e-3, rtol 1e-2
(fp32 accumulation, output rounded to the input dtype); fp32 inputs: 1e-5/1e-5.
Addressing through the block table is checked bit-exactly.
"""
import sys

import numpy as np
import pytest
import torch

import decode_attention_13_amd as fd
import oracle
from decode_attention_13_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": (1e-5, 1e-5), "f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2)}
DT = inputs.DTYPES


def announce(msg: str) -> None:
    """Name the case on the real stderr before its GPU step (survives a lost box)."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    assert fd.device_num_cus() > 0
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def assert_close(got, ref, dtype: str, what: str = ""):
    got = got.detach().to(torch.float64).cpu().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    msg = (f"{what}: max|err| {err.max():.3e}, max rel {rel.max():.3e}, "
           f"{int(bad.sum())}/{bad.size} outside atol {atol} + rtol {rtol}")
    assert not bad.any(), msg
    return err.max()


U32 = 2.0 ** -24  # fp32 unit roundoff
D = 128


def lse_atol(q_row, keys, scale: float) -> float:
    """Bound on |lse_gpu - lse| for one split, from the kernel's fp32 arithmetic.

    Each score is a D-term fp32 dot product of exactly representable products, off
    by at most gamma_D * |scale| * sum_d |q_d k_td| (gamma_D = D u / (1 - D u),
    u = 2^-24), and is scaled once more in fp32 (u |s|); a log-sum-exp moves by at
    most its largest score error. The running sum l of L terms 2^(x - m) (each from
    v_exp_f32, within 1 ulp) is off by a relative (L + 2) u, so ln l by that much;
    m + log2 l and the final multiplication by ln 2 add 3 u |lse|.
    """
    q = np.asarray(q_row, np.float64)
    k = np.asarray(keys, np.float64)
    L = k.shape[0]
    if L == 0:
        return 0.0
    dots = np.abs(k) @ np.abs(q) * abs(scale)
    s = k @ q * scale
    m = s.max()
    lse = m + np.log(np.exp(s - m).sum())
    gamma = D * U32 / (1 - D * U32)
    return float(gamma * dots.max() + U32 * np.abs(s).max() + (L + 2) * U32 + 3 * U32 * abs(lse))


def assert_lse_close(got, ref, atols, what=""):
    got = np.asarray(got.detach().cpu().numpy() if hasattr(got, "detach") else got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= np.asarray(atols))
    assert not bad.any(), f"{what}: lse max|err| {err.max():.3e}, {int(bad.sum())}/{bad.size} above the fp32 bound"


def _f64(x):
    return x.detach().to(torch.float64).numpy() if hasattr(x, "detach") else np.asarray(x, np.float64)


def split_lse_atols(q_row, k_rows, scale, bounds):
    """lse_atol of every split [a, b) of one head's key rows k_rows [L, D]."""
    return [lse_atol(q_row, k_rows[a:b], scale) for a, b in bounds]


def poisoned_workspace(nbytes: int, dev) -> torch.Tensor:
    """A workspace filled with NaN except its counter block, which every call needs
    zero on first use: a partial the call did not write shows up as NaN."""
    ws = torch.full((max(nbytes, fd.binding.WS_COUNTER_BYTES) // 4 + 1,), float("nan"), dtype=torch.float32,
                    device=dev).view(torch.uint8)
    ws[:fd.binding.WS_COUNTER_BYTES].zero_()
    return ws


def to_dev(d: dict, dev) -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_single(d, dev, opt=None, ws=None):
    g = to_dev(d, dev)
    o = fd.fd_decode(g["q"], g["k"], g["v"], scale=d["scale"], opt=opt, ws=ws)
    torch.cuda.synchronize()
    return o


def run_paged(d, dev, opt=None, ws=None, block_table=None):
    g = to_dev(d, dev)
    bt = block_table.to(dev) if block_table is not None else g["block_table"]
    o = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], bt, g["seq_lens"], d["page_size"],
                           scale=d["scale"], max_seq_len=d["max_seq_len"], total_kv=d["total_kv"], opt=opt, ws=ws)
    torch.cuda.synchronize()
    return o


# ------------------------------------------------------------------ pins on the GPU


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example(dtype, device):
    """Scores [1, 3 | 2, 5] and scalar values [10, 20 | 30, 40] embedded at D = 128
    (q = e_0, k[t, 0] = s_t): every output element is 36.8806 (the page's 36.88)."""
    announce(f"worked example {dtype}")
    s = [1.0, 3.0, 2.0, 5.0]
    vals = [10.0, 20.0, 30.0, 40.0]
    q = torch.zeros(1, 128)
    q[0, 0] = 1
    k = torch.zeros(4, 1, 128)
    k[:, 0, 0] = torch.tensor(s)
    v = torch.tensor(vals)[:, None, None].expand(4, 1, 128).contiguous()
    d = {"q": q.to(DT[dtype]), "k": k.to(DT[dtype]), "v": v.to(DT[dtype]), "scale": 1.0}
    o = run_single(d, device)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], 1.0)
    assert abs(ref[0, 0] - 36.880566) < 1e-6
    assert_close(o, ref, dtype, "worked example")


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_single_key_is_bit_exact(dtype, kernel, device):
    """S = 1: p = 1, l = 1, so o must equal v_0 bit for bit (also through a paged table).
    With 4 query heads per KV head, 16-bit inputs take the matrix-core kernel by default."""
    announce(f"single key {dtype} {kernel}")
    opt = fd.options(kernel=kernel)
    d = inputs.single_inputs(8, 2, 1, 128, dtype, 31)
    o = run_single(d, device, opt=opt)
    want = d["v"][0].repeat_interleave(4, dim=0)
    assert torch.equal(o.cpu(), want)
    p = inputs.paged_inputs(3, 8, 2, 128, dtype, 16, [1, 1, 1], 32)
    o = run_paged(p, device, opt=opt)
    for b in range(3):
        page = int(p["block_table"][b, 0])
        assert torch.equal(o[b].cpu(), p["v_cache"][page, 0].repeat_interleave(4, dim=0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_keys_give_mean(dtype, device):
    announce(f"identical keys {dtype}")
    d = inputs.single_inputs(4, 4, 777, 128, dtype, 41)
    d["k"] = d["k"][:1].expand(777, 4, 128).contiguous()
    o = run_single(d, device)
    mean = d["v"].to(torch.float64).mean(dim=0).numpy()
    assert_close(o, mean, dtype, "mean of V")


# ------------------------------------------------------------------ the five workloads


def test_workload_f32_h8_s512(device):
    w = inputs.WORKLOADS["decode_f32_h8_s512"]
    announce(f"{w.name}")
    d = w.make()
    o = run_single(d, device)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    assert_close(o, ref, "f32", w.name)


def test_workload_bf16_h32_s4096(device):
    w = inputs.WORKLOADS["decode_bf16_h32_s4096"]
    announce(f"{w.name}")
    d = w.make()
    o = run_single(d, device)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    assert_close(o, ref, "bf16", w.name)


@pytest.fixture(scope="module")
def long_peaked():
    return inputs.WORKLOADS["decode_bf16_h32_s131072_peaked"].make()


def test_workload_bf16_h32_s131072_peaked(device, long_peaked):
    """Full size, the launch the benchmark times; all 32 heads against the oracle."""
    d = long_peaked
    announce("decode_bf16_h32_s131072_peaked")
    o = run_single(d, device)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    assert_close(o, ref, "bf16", "s131072 all heads")


def test_partials_of_long_peaked(device, long_peaked):
    """The split kernel alone: the workspace partials (normalised O_s, natural-log lse_s)
    against the oracle's per-split definition, for two heads."""
    d = long_peaked
    plan = fd.decode_plan(32, 32, d["S"], "bf16")
    assert plan["merge"] != 0
    ws = fd.new_workspace(plan["workspace_bytes"], device)
    announce(f"s131072 partials chunk {plan['chunk']} splits {plan['num_splits']}")
    run_single(d, device, ws=ws)
    ws_o, ws_lse = fd.workspace_views(ws, plan, 1, 32)
    bounds = kernel_split_bounds(d["S"], plan["chunk"])
    assert len(bounds) == plan["num_splits"]
    for h in (3, 27):
        O_s, lse_s = oracle.split_partials(d["q"], d["k"], d["v"], d["scale"], plan["chunk"], heads=[h],
                                           bounds=bounds)
        assert_close(ws_o[0, h], O_s[0], "bf16", f"partials head {h}")
        atols = split_lse_atols(_f64(d["q"][h]), _f64(d["k"][:, h]), d["scale"], bounds)
        assert_lse_close(ws_lse[0, h], lse_s[0], atols, f"partials head {h}")


def kernel_split_bounds(L: int, chunk: int) -> list:
    """Token ranges of the library's splits of a contiguous cache (include/fd.h,
    workspace layout): max(1, floor(L / chunk)) splits, the last one running to L."""
    n = max(1, L // chunk) if L > 0 else 0
    return [(s * chunk, L if s == n - 1 else (s + 1) * chunk) for s in range(n)]


def paged_split_bounds(L: int, chunk: int) -> list:
    """Token ranges of the library's splits of a paged sequence: ceil(L / chunk)
    splits, the last one holding the remainder."""
    return [(s, min(s + chunk, L)) for s in range(0, L, chunk)]


def paged_item_order(lens, chunk: int) -> list:
    """(sequence, split) of every item of a paged batch in the library's item order:
    the full splits sequence by sequence, then the remainder splits by decreasing
    size (ties by sequence), the empty sequences last."""
    items = [(b, s) for b, L in enumerate(lens) for s in range(L // chunk)]
    rem = [(L % chunk if L else 0, b) for b, L in enumerate(lens) if L % chunk or L == 0]
    rem.sort(key=lambda kb: (-kb[0], kb[1]))
    return items + [(b, lens[b] // chunk) for _, b in rem]


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
def test_partials_last_split_takes_the_remainder(kernel, device):
    """S = 1000 with a 64-token stride: 15 splits, the last one 104 tokens long; the
    workspace partials against the oracle over the same token ranges."""
    d = inputs.single_inputs(8, 2, 1000, 128, "bf16", 95, peak_frac=0.01)
    opt = fd.options(force_chunk=64, kernel=kernel)
    plan = fd.decode_plan(8, 2, 1000, "bf16", 0, opt)
    assert plan["num_splits"] == 15 and plan["merge"] != 0
    ws = fd.new_workspace(plan["workspace_bytes"], device)
    announce(f"remainder partials {kernel}")
    o = run_single(d, device, opt=opt, ws=ws)
    ws_o, ws_lse = fd.workspace_views(ws, plan, 1, 8)
    bounds = kernel_split_bounds(1000, 64)
    assert bounds[-1] == (896, 1000)
    O_s, lse_s = oracle.split_partials(d["q"], d["k"], d["v"], d["scale"], 64, bounds=bounds)
    for h in range(8):
        assert_close(ws_o[0, h], O_s[h], "bf16", f"partials head {h}")
        atols = split_lse_atols(_f64(d["q"][h]), _f64(d["k"][:, h // 4]), d["scale"], bounds)
        assert_lse_close(ws_lse[0, h], lse_s[h], atols, f"partials head {h}")
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    assert_close(o, ref, "bf16", "merged")


def _sample_pairs(B, H, lens, n, seed):
    rng = np.random.default_rng(seed)
    order = np.argsort(lens)
    bs = sorted(set([int(order[0]), int(order[-1])] + rng.choice(B, size=n, replace=False).tolist()))
    return [(b, int(h)) for b in bs for h in rng.choice(H, size=3, replace=False)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["paged_gqa4_bf16_b64_s1k-8k", "paged_gqa8_f16_b128_s256-64k"])
def test_paged_workloads(name, device):
    """Full size in the benchmark's launch (matrix-core kernel, the work list for the
    GQA8 batch), then the vector-ALU kernel forced; every (sequence, head) row
    against the oracle."""
    w = inputs.WORKLOADS[name]
    announce(f"{name} (generating inputs)")
    d = w.make()
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           d["page_size"], d["scale"])
    for kernel in ("auto", "valu"):
        announce(f"{name} run {kernel}")
        o = run_paged(d, device, opt=fd.options(kernel=kernel))
        assert_close(o, ref, w.dtype, f"{name} {kernel}")
    announce(f"{name} grid launch")
    auto = fd.paged_plan(w.B, w.H, w.Hkv, w.dtype, 16, d["max_seq_len"], d["total_kv"])
    assert auto["persistent"] == 1
    og = run_paged(d, device, opt=fd.options(launch="grid"))
    assert torch.equal(og, run_paged(d, device))  # the same splits claimed or one per workgroup


# ------------------------------------------------------------------ invariance and tails


@pytest.mark.parametrize("H,Hkv,kernel", [(8, 8, "auto"), (8, 8, "mfma"), (32, 4, "auto"), (32, 4, "valu")])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_split_count_and_chunk_invariance(dtype, H, Hkv, kernel, device):
    """Any split count or chunk, either split kernel: the same result within tolerance
    (a 4099-token cache with peaked keys)."""
    if dtype == "f32" and kernel == "mfma":
        pytest.skip("the matrix-core kernel takes 16-bit inputs")
    d = inputs.single_inputs(H, Hkv, 4099, 128, dtype, 51, peak_frac=0.01)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    for n, c in [(1, 0), (2, 0), (3, 0), (7, 0), (64, 0), (0, 0), (0, 64), (0, 192), (0, 1024)]:
        opt = fd.options(force_num_splits=n, force_chunk=c, kernel=kernel)
        plan = fd.decode_plan(H, Hkv, 4099, dtype, 0, opt)
        announce(f"invariance {dtype} H{H}/{Hkv} k{plan['kernel']} chunk {plan['chunk']} splits {plan['num_splits']}")
        o = run_single(d, device, opt=opt)
        assert_close(o, ref, dtype, f"kernel {plan['kernel']} chunk {plan['chunk']}")


@pytest.mark.parametrize("S", [0, 1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 255, 257, 1000, 4097])
def test_ragged_lengths(S, device):
    announce(f"ragged S={S}")
    d = inputs.single_inputs(8, 2, S, 128, "bf16", 60 + S)
    for opt in (None, fd.options(force_chunk=64), fd.options(kernel="valu"),
                fd.options(force_chunk=64, kernel="valu")):
        o = run_single(d, device, opt=opt)
        ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
        assert_close(o, ref, "bf16", f"S={S}")


@pytest.mark.parametrize("kernel", ["auto", "valu", "mfma"])
@pytest.mark.parametrize("H,Hkv", [(4, 4), (8, 4), (16, 4), (16, 2), (12, 4), (12, 2), (7, 1), (32, 4),
                                   (16, 1), (64, 2)])
def test_head_groups(H, Hkv, kernel, device):
    """Group sizes 1, 2, 4, 8, 3, 6, 7, 16, 32: each q head reads KV head h // (H / Hkv)."""
    announce(f"heads H={H} Hkv={Hkv} {kernel}")
    d = inputs.single_inputs(H, Hkv, 700, 128, "bf16", 70 + H * 10 + Hkv)
    o = run_single(d, device, opt=fd.options(force_chunk=256, kernel=kernel))
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    assert_close(o, ref, "bf16", f"H={H} Hkv={Hkv} {kernel}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("H", [1, 2, 3, 5, 6, 12, 32])
def test_mha_packed_kv_heads(H, dtype, device):
    """H = Hkv: the vector-ALU kernel reads 2 adjacent KV heads per workgroup when
    Hkv is even (1 otherwise); ragged 777 tokens, strides 64 and automatic."""
    d = inputs.single_inputs(H, H, 777, 128, dtype, 400 + H)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    for opt in (None, fd.options(force_chunk=64), fd.options(force_num_splits=1)):
        plan = fd.decode_plan(H, H, 777, dtype, 0, opt)
        assert plan["kv_heads_per_group"] == (2 if H % 2 == 0 else 1)
        announce(f"mha packed H={H} {dtype} hp={plan['kv_heads_per_group']} chunk {plan['chunk']}")
        assert_close(run_single(d, device, opt=opt), ref, dtype, f"H={H} chunk {plan['chunk']}")


@pytest.mark.parametrize("ps", [1, 16])
def test_paged_mha_packed_is_bit_exact(ps, device):
    """Paged MHA (6 heads: packed in pairs): shuffled pages == in-order pages bit for bit,
    NaN poison unread, and the oracle within tolerance."""
    lens = [1, 17, 1000, 3000]
    kA, vA, tA, kB, vB, tB = _pools(lens, 6, ps, "bf16", 410 + ps)
    q = inputs.normal(np.random.SeedSequence(411), (4, 6, 128), "bf16")
    L = torch.tensor(lens, dtype=torch.int32)
    outs = []
    for kc, vc, t in ((kA, vA, tA), (kB, vB, tB)):
        announce(f"paged mha packed ps={ps}")
        o = fd.fd_paged_decode(q.to(device), kc.to(device), vc.to(device), t.to(device), L.to(device), ps,
                               scale=0.09, max_seq_len=max(lens), total_kv=sum(lens),
                               opt=fd.options(force_chunk=256))
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    ref, _ = oracle.paged_decode_attention(q, kB, vB, tB, L, ps, 0.09)
    assert_close(outs[1], ref, "bf16", f"paged mha ps={ps}")


# ------------------------------------------------------------------ paged addressing


def _pools(lens, Hkv, ps, dtype, seed):
    """The same tokens stored (a) in order with an identity table and (b) on shuffled
    pages, every slot past L_b and three spare pages filled with NaN."""
    B = len(lens)
    rng = np.random.default_rng(seed)
    counts = [-(-L // ps) for L in lens]
    P = sum(counts)
    perm = rng.permutation(P)
    nan_pool = torch.full((P + 3, ps, Hkv, 128), float("nan"), dtype=DT[dtype])
    kA, vA, kB, vB = nan_pool.clone(), nan_pool.clone(), nan_pool.clone(), nan_pool.clone()
    tA = torch.full((B, max(counts)), -1, dtype=torch.int32)
    tB = tA.clone()
    nxt = 0
    for b, L in enumerate(lens):
        kt = inputs.normal(np.random.SeedSequence([seed, b, 0]), (L, Hkv, 128), dtype)
        vt = inputs.normal(np.random.SeedSequence([seed, b, 1]), (L, Hkv, 128), dtype)
        for j in range(counts[b]):
            n = min(ps, L - j * ps)
            tA[b, j] = nxt
            tB[b, j] = int(perm[nxt])
            kA[nxt, :n] = kt[j * ps:j * ps + n]
            vA[nxt, :n] = vt[j * ps:j * ps + n]
            kB[int(perm[nxt]), :n] = kt[j * ps:j * ps + n]
            vB[int(perm[nxt]), :n] = vt[j * ps:j * ps + n]
            nxt += 1
    return kA, vA, tA, kB, vB, tB


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("ps", [1, 4, 16, 64, 256, 1024])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_paged_addressing_is_bit_exact(ps, dtype, kernel, device):
    """Shuffled table over a scattered pool == identity table over in-order pages, bit
    for bit; NaN in tail slots and unreferenced pages never reaches the output. Lengths
    {1, 17, 1000, 4096} are those of the paged GQA harness on "FlashAttention 与推理算子"."""
    lens = [1, 17, 1000, 4096]
    B, H, Hkv = 4, 32, 8
    kA, vA, tA, kB, vB, tB = _pools(lens, Hkv, ps, dtype, 80 + ps)
    q = inputs.normal(np.random.SeedSequence(81), (B, H, 128), dtype)
    L = torch.tensor(lens, dtype=torch.int32)
    scale = inputs.default_scale(128)
    outs = []
    for kc, vc, t in ((kA, vA, tA), (kB, vB, tB)):
        announce(f"paged bit-exact ps={ps} {dtype} {kernel}")
        o = fd.fd_paged_decode(q.to(device), kc.to(device), vc.to(device), t.to(device), L.to(device), ps,
                               scale=scale, max_seq_len=max(lens), total_kv=sum(lens),
                               opt=fd.options(force_chunk=512, kernel=kernel))
        torch.cuda.synchronize()
        outs.append(o.cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    ref, _ = oracle.paged_decode_attention(q, kB, vB, tB, L, ps, scale)
    assert_close(outs[1], ref, dtype, f"paged ps={ps}")


def test_paged_empty_and_clamped_sequences(device):
    """L_b = 0 gives zeros; the rest of the batch is unaffected."""
    lens = [0, 5, 0, 300]
    d = inputs.paged_inputs(4, 8, 2, 128, "bf16", 16, lens, 90)
    announce("paged empty sequences")
    for opt in (None, fd.options(force_chunk=64)):
        o = run_paged(d, device, opt=opt)
        assert torch.equal(o[0].cpu(), torch.zeros(8, 128, dtype=torch.bfloat16))
        assert torch.equal(o[2].cpu(), torch.zeros(8, 128, dtype=torch.bfloat16))
        ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                               d["seq_lens"], 16, d["scale"])
        assert_close(o, ref, "bf16", "paged with empty sequences")


def test_paged_split_invariance(device):
    lens = [4097, 1, 3000, 64, 8191]
    d = inputs.paged_inputs(5, 16, 2, 128, "f16", 16, lens, 91)
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"])
    for opt in (None, fd.options(force_chunk=64), fd.options(force_chunk=1024), fd.options(force_num_splits=3)):
        plan = fd.paged_plan(5, 16, 2, "f16", 16, max(lens), sum(lens), 0, opt)
        announce(f"paged invariance chunk {plan['chunk']}")
        o = run_paged(d, device, opt=opt)
        assert_close(o, ref, "f16", f"paged chunk {plan['chunk']}")


@pytest.mark.parametrize("H,Hkv,S,chunk", [(1, 1, 131072, 128), (2, 1, 65600, 64), (4, 2, 40000, 1024)])
def test_many_splits(H, Hkv, S, chunk, device):
    """Up to 2048 splits per head: the merge kernel splits the work across its waves."""
    d = inputs.single_inputs(H, Hkv, S, 128, "bf16", 300 + S, peak_frac=0.01)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    for kernel in ("valu", "mfma"):
        announce(f"many splits H={H} S={S} chunk={chunk} {kernel}")
        o = run_single(d, device, opt=fd.options(force_chunk=chunk, kernel=kernel))
        assert_close(o, ref, "bf16", f"H={H} S={S} chunk={chunk} {kernel}")


def test_workspace_reuse_across_plans(device):
    """One workspace (filled with NaN but for its zeroed counter block) serves calls of
    different plans in any order, fused and merge-kernel ones alike: nothing is read
    from it that the same call did not write, and every call leaves the counters zero."""
    cases = [inputs.single_inputs(8, 8, S, 128, "bf16", 200 + S) for S in (4099, 1000, 8191)]
    refs = [oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])[0] for d in cases]
    plans = [(i, c) for i in range(3) for c in (64, 256, 1024)]
    need = max(fd.decode_plan(8, 8, cases[i]["S"], "bf16", 0, fd.options(force_chunk=c))["workspace_bytes"]
               for i, c in plans)
    ws = poisoned_workspace(need, device)
    rng = np.random.default_rng(7)
    for k in rng.permutation(len(plans)).tolist() + rng.permutation(len(plans)).tolist():
        i, c = plans[k]
        announce(f"workspace reuse S={cases[i]['S']} chunk={c}")
        o = run_single(cases[i], device, opt=fd.options(force_chunk=c), ws=ws)
        assert_close(o, refs[i], "bf16", f"S={cases[i]['S']} chunk={c}")


def test_paged_many_sequences_ragged_splits(device):
    """96 sequences of 1..6000 tokens: single-split sequences written directly, the
    others merged, in one call."""
    lens = np.random.default_rng(11).integers(1, 6000, size=96).tolist()
    d = inputs.paged_inputs(96, 16, 4, 128, "bf16", 16, lens, 12)
    pairs = [(b, h) for b in range(0, 96, 7) for h in (0, 5, 15)]
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"], pairs=pairs)
    for c in (64, 512, 4096):
        announce(f"paged many sequences chunk={c}")
        o = run_paged(d, device, opt=fd.options(force_chunk=c))
        got = torch.stack([o[b, h] for b, h in pairs])
        assert_close(got, ref, "bf16", f"chunk={c}")


def _ragged_batch(B, seed, lo=1, hi=6000):
    rng = np.random.default_rng(seed)
    lens = np.exp(rng.uniform(np.log(lo), np.log(hi), B)).astype(int).tolist()
    lens[3] = 0  # an empty sequence
    return lens, inputs.paged_inputs(B, 32, 8, 128, "bf16", 16, lens, seed)


@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_work_list_matches_grid(kernel, device):
    """A batch far shorter than its longest sequence, three launches of the same
    splits: numbered items (work list, total_kv given), the full (split, sequence)
    grid (total_kv unknown), and one workgroup per resident slot claiming the items
    (persistent). Same splits, same arithmetic: bit-identical outputs, and the oracle
    agrees."""
    lens, d = _ragged_batch(48, 420)
    total = sum(lens)
    opts = {"list": fd.options(force_chunk=256, kernel=kernel, launch="grid"),
            "grid": fd.options(force_chunk=256, kernel=kernel, launch="grid"),
            "persistent": fd.options(force_chunk=256, kernel=kernel)}
    totals = {"list": total, "grid": 0, "persistent": total}
    p_list = fd.paged_plan(48, 32, 8, "bf16", 16, max(lens), total, 0, opts["list"])
    p_grid = fd.paged_plan(48, 32, 8, "bf16", 16, max(lens), 0, 0, opts["grid"])
    p_pers = fd.paged_plan(48, 32, 8, "bf16", 16, max(lens), total, 0, opts["persistent"])
    assert p_list["work_list"] == 1 and p_grid["work_list"] == 0 and p_pers["persistent"] == 1
    assert p_list["grid_y"] == 48 + total // 256
    outs = []
    for name in ("list", "grid", "persistent"):
        announce(f"work list {kernel} {name}")
        g = to_dev(d, device)
        outs.append(fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                       scale=d["scale"], max_seq_len=max(lens), total_kv=totals[name],
                                       opt=opts[name]).cpu())
        torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert torch.all(outs[0][3] == 0)
    pairs = _sample_pairs(48, 32, np.array(lens), 6, 421)
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"], pairs=pairs)
    assert_close(torch.stack([outs[0][b, h] for b, h in pairs]), ref, "bf16", f"work list {kernel}")


def test_work_list_short_total_is_nan(device):
    """total_kv below the true sum, work-list grid: the splits past the shortened work
    list have no workgroup, and exactly the sequences that own one come out NaN; every
    other sequence is bit-identical to the full-grid result. A persistent launch
    numbers the items on the device and gets every sequence right."""
    lens, d = _ragged_batch(48, 430)
    opt = fd.options(force_chunk=256, launch="grid")
    # The work-list grid holds B + total_kv // chunk items, taken in the library's
    # item order; a total_kv that leaves out the five smallest remainder splits
    # (the empty sequence's item among them) cuts exactly those five sequences.
    order = paged_item_order(lens, 256)
    short = (len(order) - 5 - 48) * 256
    plan = fd.paged_plan(48, 32, 8, "bf16", 16, max(lens), short, 0, opt)
    assert plan["work_list"] == 1 and plan["grid_y"] == len(order) - 5
    missing = sorted({b for b, _ in order[plan["grid_y"]:]})
    assert len(missing) == 5 and 3 in missing
    g = to_dev(d, device)
    outs = []
    for tk in (short, 0):
        announce(f"work list short total_kv={tk}")
        outs.append(fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                       scale=d["scale"], max_seq_len=max(lens), total_kv=tk, opt=opt).cpu())
        torch.cuda.synchronize()
    for b in range(48):
        if b in missing:
            assert torch.isnan(outs[0][b].float()).all(), b
        else:
            assert torch.equal(outs[0][b], outs[1][b]), b
    pers = fd.options(force_chunk=256, launch="persistent")
    assert fd.paged_plan(48, 32, 8, "bf16", 16, max(lens), short, 0, pers)["persistent"] == 1
    announce("persistent, short total_kv")
    o = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                           scale=d["scale"], max_seq_len=max(lens), total_kv=short, opt=pers).cpu()
    torch.cuda.synchronize()
    assert torch.equal(o, outs[1])


def test_persistent_counters_return_to_zero(device):
    """Persistent launches of different sizes on one workspace (a KV-head group of 2
    heads on one short sequence: 2 units; a 12-sequence batch; a 40-sequence batch),
    repeated: each output is bit-identical to the one-item-per-workgroup grid, and
    every claim and exit counter is back at zero after every call."""
    cases = []
    for B, H, Hkv, lens, seed in ((1, 8, 2, [100], 431), (12, 32, 8, None, 432), (40, 32, 8, None, 433)):
        if lens is None:
            lens = np.random.default_rng(seed).integers(0, 3000, B).tolist()
        d = inputs.paged_inputs(B, H, Hkv, 128, "bf16", 16, lens, seed)
        grid = fd.options(force_chunk=256, launch="grid")
        g = to_dev(d, device)
        ref = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                 scale=d["scale"], max_seq_len=max(lens), total_kv=sum(lens), opt=grid).cpu()
        cases.append((B, H, Hkv, lens, g, d, ref))
    pers = fd.options(force_chunk=256, launch="persistent")
    size = max(fd.paged_plan(B, H, Hkv, "bf16", 16, max(lens), sum(lens), 0, pers)["workspace_bytes"]
               for B, H, Hkv, lens, _, _, _ in cases)
    ws = fd.new_workspace(size, device)
    for rep in range(3):
        for B, H, Hkv, lens, g, d, ref in cases:
            plan = fd.paged_plan(B, H, Hkv, "bf16", 16, max(lens), sum(lens), 0, pers)
            assert plan["persistent"] == 1
            announce(f"persistent counters rep {rep} B={B} grid_x={plan['grid_x']}")
            o = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                   scale=d["scale"], max_seq_len=max(lens), total_kv=sum(lens), opt=pers, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(o.cpu(), ref), (rep, B)
            assert torch.all(ws[:fd.binding.WS_COUNTER_BYTES] == 0), (rep, B)


def test_workspace_too_small_is_rejected(device):
    d = to_dev(inputs.single_inputs(8, 8, 4096, 128, "bf16", 95), device)
    plan = fd.decode_plan(8, 8, 4096, "bf16", 0, fd.options(force_num_splits=4))
    ws = fd.new_workspace(plan["workspace_bytes"] - 4, device)
    with pytest.raises(fd.FdError) as e:
        fd.fd_decode(d["q"], d["k"], d["v"], scale=0.1, ws=ws, opt=fd.options(force_num_splits=4))
    assert e.value.name == "FD_ERR_WORKSPACE"


@pytest.mark.parametrize("B", [1024, 1025])
def test_paged_largest_work_list_batch(B, device):
    """The work list holds at most 1024 sequences (their offsets live in LDS): a
    batch of 1024 short ragged sequences takes it, 1025 falls back to the grid.
    Both match the oracle on sampled rows, the last sequences included, and the
    1024-sequence batch is bit-identical to its own full-grid run."""
    rng = np.random.default_rng(900 + B)
    lens = np.clip(np.round(np.exp(rng.uniform(0.0, np.log(2000), B))), 1, 2000).astype(int).tolist()
    d = inputs.paged_inputs(B, 8, 2, 128, "bf16", 16, lens, 901 + B)
    opt = fd.options(force_chunk=64)
    total = sum(lens)
    plan = fd.paged_plan(B, 8, 2, "bf16", 16, max(lens), total, 0, opt)
    assert plan["work_list"] == (1 if B <= 1024 else 0)
    announce(f"paged largest work-list batch B={B}")
    o = run_paged(d, device, opt=opt)
    bs = sorted(set(list(range(0, B, 97)) + [B - 2, B - 1]))
    pairs = [(b, h) for b in bs for h in (0, 7)]
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"], pairs=pairs)
    assert_close(torch.stack([o[b, h] for b, h in pairs]), ref, "bf16", f"B={B}")
    if plan["work_list"]:
        g = to_dev(d, device)
        announce(f"paged largest work-list batch B={B}, full grid")
        og = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                                scale=d["scale"], max_seq_len=max(lens), total_kv=0, opt=opt)
        torch.cuda.synchronize()
        assert torch.equal(o.cpu(), og.cpu())


@pytest.mark.parametrize("H,Hkv", [(8, 8), (32, 4)])
@pytest.mark.parametrize("scale", [float(np.float32(-0.3)), 0.0, float(np.float32(2.5))])
def test_decode_any_finite_scale(H, Hkv, scale, device):
    """The online softmax takes scores of any sign and size: a negative scale, a
    zero one (every weight equal: the mean of V) and a large one (a peaked
    softmax), on both split kernels (MHA on the vector ALUs, GQA4 on the matrix
    cores) and through the block table."""
    d = inputs.single_inputs(H, Hkv, 1000, 128, "bf16", 520 + H)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], scale)
    g = to_dev(d, device)
    for kernel in ("auto", "valu"):
        announce(f"decode scale={scale} H={H} Hkv={Hkv} {kernel}")
        o = fd.fd_decode(g["q"], g["k"], g["v"], scale=scale, opt=fd.options(force_chunk=256, kernel=kernel))
        torch.cuda.synchronize()
        assert_close(o, ref, "bf16", f"scale={scale} {kernel}")
    # the same tokens as one paged sequence (pages of 16 in order)
    pages = -(-1000 // 16)
    kp = torch.zeros(pages * 16, Hkv, 128, dtype=d["k"].dtype)
    vp = torch.zeros_like(kp)
    kp[:1000], vp[:1000] = d["k"], d["v"]
    table = torch.arange(pages, dtype=torch.int32).reshape(1, pages)
    announce(f"paged decode scale={scale} H={H} Hkv={Hkv}")
    o = fd.fd_paged_decode(g["q"].reshape(1, H, 128), kp.reshape(pages, 16, Hkv, 128).to(device),
                           vp.reshape(pages, 16, Hkv, 128).to(device), table.to(device),
                           torch.tensor([1000], dtype=torch.int32, device=device), 16, scale=scale,
                           max_seq_len=1000, total_kv=1000, opt=fd.options(force_chunk=256))
    torch.cuda.synchronize()
    assert_close(o[0], ref, "bf16", f"paged scale={scale}")


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("H,Hkv", [(64, 4), (64, 2), (48, 3)])
def test_paged_large_head_groups(H, Hkv, kernel, device):
    """Paged batches with 16 and 32 query heads per KV head (the matrix-core kernel
    splits a group over several workgroups) and 16 over an odd KV-head count, on
    ragged lengths that give one-split and many-split sequences."""
    lens = [5, 300, 1500, 4000]
    d = inputs.paged_inputs(len(lens), H, Hkv, 128, "f16", 16, lens, 930 + H + Hkv)
    announce(f"paged large groups H={H} Hkv={Hkv} {kernel}")
    o = run_paged(d, device, opt=fd.options(force_chunk=512, kernel=kernel))
    pairs = [(b, h) for b in range(len(lens)) for h in (0, H // 2 - 1, H // 2, H - 1)]
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"], pairs=pairs)
    assert_close(torch.stack([o[b, h] for b, h in pairs]), ref, "f16", f"H={H} Hkv={Hkv} {kernel}")


def test_paged_long_sequence(device):
    """A 128k-token sequence beside a 100-token one in a paged GQA4 batch (8192
    pages of 16 tokens, shuffled): the planner's largest paged strides, table
    slices staged across many pages, on sampled heads of both sequences."""
    lens = [131072, 100]
    d = inputs.paged_inputs(2, 32, 8, 128, "bf16", 16, lens, 940)
    plan = fd.paged_plan(2, 32, 8, "bf16", 16, max(lens), sum(lens), 0)
    announce(f"paged long sequence plan chunk={plan['chunk']} splits={plan['num_splits']}")
    o = run_paged(d, device)
    pairs = [(b, h) for b in range(2) for h in (0, 13, 31)]
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"], pairs=pairs)
    assert_close(torch.stack([o[b, h] for b, h in pairs]), ref, "bf16", "paged 128k")


# ------------------------------------------------------------------ paged partials, sweep lengths


@pytest.mark.parametrize("launch", ["grid", "persistent"])
@pytest.mark.parametrize("work_list", [True, False])
@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_paged_partials(kernel, work_list, launch, device):
    """The paged split kernels alone: ws_o / ws_lse of every split of every (sequence,
    head) of a ragged batch on shuffled pages, against the oracle's paged partials over
    the library's token ranges; with the numbered work list (total_kv given) and with
    the full grid, and as one workgroup per resident slot claiming the items. The
    workspace starts NaN-filled, so an unwritten partial shows."""
    lens = [5, 300, 1500, 4000, 2049, 0, 64, 3333]
    B, H, Hkv, chunk = len(lens), 32, 8, 256
    d = inputs.paged_inputs(B, H, Hkv, 128, "bf16", 16, lens, 960)
    opt = fd.options(force_chunk=chunk, kernel=kernel, launch=launch)
    total = sum(lens) if work_list else 0
    plan = fd.paged_plan(B, H, Hkv, "bf16", 16, max(lens), total, 0, opt)
    assert plan["work_list"] == int(work_list) and plan["merge"] == 1 and plan["chunk"] == chunk
    assert plan["persistent"] == (launch == "persistent")
    ws = poisoned_workspace(plan["workspace_bytes"], device)
    g = to_dev(d, device)
    announce(f"paged partials {kernel} work_list={work_list} {launch}")
    o = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"], g["seq_lens"], 16,
                           scale=d["scale"], max_seq_len=max(lens), total_kv=total, opt=opt, ws=ws)
    torch.cuda.synchronize()
    ws_o, ws_lse = fd.workspace_views(ws, plan, B, H)
    checked = 0
    for b, L in enumerate(lens):
        bounds = paged_split_bounds(L, chunk)
        if len(bounds) <= 1:
            continue  # one split: written to o directly
        kb = oracle.gather_pages(d["k_cache"], d["block_table"][b], L, 16)
        for h in range(H):
            O_s, lse_s = oracle.paged_split_partials(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                                     d["seq_lens"], 16, d["scale"], chunk, b, h, bounds=bounds)
            n = len(bounds)
            assert_close(ws_o[b, h, :n], O_s, "bf16", f"partials b={b} h={h}")
            atols = split_lse_atols(_f64(d["q"][b, h]), _f64(kb[:, h // 4]), d["scale"], bounds)
            assert_lse_close(ws_lse[b, h, :n], lse_s, atols, f"partials b={b} h={h}")
            checked += n
    assert checked > 0
    ref, _ = oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                           16, d["scale"])
    assert_close(o, ref, "bf16", f"paged partials merged {kernel}")


SWEEP_HEADS = [0, 1, 14, 30, 31]  # both heads of the first and the last KV-head pair


@pytest.mark.timeout(600)
@pytest.mark.parametrize("S", [8192, 16384, 32768, 65536, 131073])
def test_sweep_length_full_size(S, device):
    """The KV-length curve the benchmark times (32 heads, bf16) at full size in its own
    launch: five heads against the oracle, every head finite; at 131073 tokens (the
    pages' odd length) the last split holds chunk + 1 tokens, and the workspace
    partials of two heads, that split included, are checked as well."""
    w = inputs.sweep_workload(S)
    d = w.make()
    plan = fd.decode_plan(32, 32, S, "bf16")
    ws = poisoned_workspace(plan["workspace_bytes"], device)
    announce(f"sweep S={S} chunk {plan['chunk']} splits {plan['num_splits']}")
    o = run_single(d, device, ws=ws)
    assert torch.isfinite(o.float()).all()
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"], heads=SWEEP_HEADS)
    assert_close(o[SWEEP_HEADS], ref, "bf16", f"S={S}")
    if S == 131073:
        bounds = kernel_split_bounds(S, plan["chunk"])
        assert plan["merge"] != 0 and bounds[-1][1] - bounds[-1][0] == plan["chunk"] + 1
        ws_o, ws_lse = fd.workspace_views(ws, plan, 1, 32)
        for h in (1, 30):
            O_s, lse_s = oracle.split_partials(d["q"], d["k"], d["v"], d["scale"], plan["chunk"], heads=[h],
                                               bounds=bounds)
            assert_close(ws_o[0, h], O_s[0], "bf16", f"S={S} partials head {h}")
            atols = split_lse_atols(_f64(d["q"][h]), _f64(d["k"][:, h]), d["scale"], bounds)
            assert_lse_close(ws_lse[0, h], lse_s[0], atols, f"S={S} partials head {h}")


# ------------------------------------------------------------------ device-data checks


@pytest.mark.parametrize("launch", ["auto", "persistent"])
@pytest.mark.parametrize("work_list", [True, False])
@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_debug_checks_report_bad_table_and_lengths(kernel, work_list, launch, device):
    """fd_options.debug_checks: a clean batch gives the same output bit for bit as
    without it; a table entry outside [0, num_pages) inside a sequence's pages, or a
    negative length, comes back as FD_ERR_BAD_DATA naming the sequence and index.
    The -1 padding past each sequence's pages is never reported. Without the checks
    the bad entry is clamped (no access leaves the cache) and the other sequences
    are unchanged."""
    lens = [5, 300, 1500, 4000]
    d = inputs.paged_inputs(4, 32, 8, 128, "bf16", 16, lens, 970)
    assert (d["block_table"] == -1).any()  # padded rows
    g = to_dev(d, device)
    total = sum(lens) if work_list else 0

    def call(debug, table=None, seq_lens=None):
        opt = fd.options(force_chunk=256, kernel=kernel, debug_checks=debug, launch=launch)
        o = fd.fd_paged_decode(g["q"], g["k_cache"], g["v_cache"], g["block_table"] if table is None else table,
                               g["seq_lens"] if seq_lens is None else seq_lens, 16, scale=d["scale"],
                               max_seq_len=max(lens), total_kv=total, opt=opt)
        torch.cuda.synchronize()
        return o.cpu()

    plan = fd.paged_plan(4, 32, 8, "bf16", 16, max(lens), total, 0,
                         fd.options(force_chunk=256, kernel=kernel, launch=launch))
    assert plan["work_list"] == int(work_list) and plan["persistent"] == (launch == "persistent")
    announce(f"debug checks {kernel} work_list={work_list} {launch}: clean")
    clean = call(False)
    assert torch.equal(call(True), clean)
    bad = d["block_table"].clone()
    bad[2, 40] = d["num_pages"] + 7
    bad_dev = bad.to(device)
    announce(f"debug checks {kernel} work_list={work_list}: bad entry")
    with pytest.raises(fd.FdError) as e:
        call(True, table=bad_dev)
    assert e.value.name == "FD_ERR_BAD_DATA" and f"block_table[2][40] = {d['num_pages'] + 7}" in str(e.value)
    neg = d["block_table"].clone()
    neg[1, 3] = -1
    with pytest.raises(fd.FdError) as e:
        call(True, table=neg.to(device))
    assert "block_table[1][3] = -1" in str(e.value)
    lens_bad = d["seq_lens"].clone()
    lens_bad[3] = -5
    announce(f"debug checks {kernel} work_list={work_list}: bad length")
    with pytest.raises(fd.FdError) as e:
        call(True, seq_lens=lens_bad.to(device))
    assert e.value.name == "FD_ERR_BAD_DATA" and "seq_lens[3] = -5" in str(e.value)
    announce(f"debug checks {kernel} work_list={work_list}: bad entry, checks off")
    o = call(False, table=bad_dev)
    for b in (0, 1, 3):
        assert torch.equal(o[b], clean[b])


# ------------------------------------------------------------------ fused merge


FUSED_CASES = [  # (H, Hkv, S, dtype, kernel, chunk); at most 64 (head, split) rows per workgroup
    (8, 8, 512, "f32", "auto", 0),        # the 512-token fp32 decode's own plan: 32 splits of 16
    (32, 32, 4096, "bf16", "auto", 0),    # the 4k decode's own plan
    (32, 32, 4099, "bf16", "auto", 256),  # ragged last split
    (32, 4, 3000, "bf16", "auto", 448),   # 8 heads per KV head on the matrix cores: 6 splits
    (32, 4, 3000, "f16", "valu", 448),    # the same on the vector ALUs (8 heads per workgroup)
    (64, 4, 2048, "bf16", "auto", 1024),  # 16 heads per workgroup, 2 splits
    (12, 3, 777, "f32", "auto", 64),      # fp32 GQA
]


@pytest.mark.parametrize("H,Hkv,S,dtype,kernel,chunk", FUSED_CASES)
def test_fused_and_kernel_merge_agree(H, Hkv, S, dtype, kernel, chunk, device):
    """The one-launch step (the last workgroup of each head slice merges) and the
    two-launch step (a merge kernel) on the same plan: both against the oracle, and
    the partials they leave in the workspace are the same bits."""
    d = inputs.single_inputs(H, Hkv, S, 128, dtype, 990 + S + H)
    ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    outs, parts = {}, {}
    for merge in ("fused", "kernel"):
        opt = fd.options(force_chunk=chunk, kernel=kernel, merge=merge)
        plan = fd.decode_plan(H, Hkv, S, dtype, 0, opt)
        assert plan["merge"] == {"fused": 2, "kernel": 1}[merge]
        ws = poisoned_workspace(plan["workspace_bytes"], device)
        announce(f"fused/kernel merge {merge} H={H} Hkv={Hkv} S={S} {dtype} splits {plan['num_splits']}")
        outs[merge] = run_single(d, device, opt=opt, ws=ws).cpu()
        assert_close(outs[merge], ref, dtype, f"{merge} merge")
        wo, wl = fd.workspace_views(ws, plan, 1, H)
        parts[merge] = (wo.cpu(), wl.cpu())
        assert torch.all(ws[:fd.binding.WS_COUNTER_BYTES] == 0)  # counters left at zero
    assert torch.equal(parts["fused"][0], parts["kernel"][0]) and torch.equal(parts["fused"][1], parts["kernel"][1])


def test_fused_merge_repeated_calls(device):
    """Forty fused calls on one workspace, alternating two inputs of the same plan:
    every output is bit-identical to the first output of its input, so no call ever
    merges a partial left by the call before it."""
    ds = [inputs.single_inputs(32, 32, 4096, 128, "bf16", 995 + i) for i in range(2)]
    gs = [to_dev(d, device) for d in ds]
    opt = fd.options(merge="fused")
    plan = fd.decode_plan(32, 32, 4096, "bf16", 0, opt)
    assert plan["merge"] == 2
    ws = fd.new_workspace(plan["workspace_bytes"], device)
    announce("fused repeated calls")
    first = [None, None]
    outs = []
    for i in range(40):
        g = gs[i % 2]
        outs.append(fd.fd_decode(g["q"], g["k"], g["v"], scale=ds[0]["scale"], ws=ws, opt=opt))
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        if first[i % 2] is None:
            first[i % 2] = o.cpu()
        assert torch.equal(o.cpu(), first[i % 2]), i
    for j, d in enumerate(ds):
        ref, _ = oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
        assert_close(first[j], ref, "bf16", f"input {j}")
