"""GPU parity of the FP8 E4M3 KV-cache entry points (fd_decode_fp8kv,
fd_paged_decode_fp8kv) against the float64 oracle over the dequantised cache.

Every E4M3 value converts exactly to f16, bf16 and fp32, so the tolerance is that
of 16-bit inputs (|gpu - ref| <= 2e-3 + 1e-2 |ref|): fp32 accumulation and the
rounding of the output to the query dtype. The decoding of the codes themselves is
checked bit for bit (one key: o is v_scale times the cached value).
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
DT = inputs.DTYPES


def announce(msg: str) -> None:
    sys.__stderr__.write(f"[gpu-case] fp8 {msg}\n")
    sys.__stderr__.flush()


@pytest.fixture(scope="module", autouse=True)
def device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    fd.lib()
    torch.cuda.set_device(0)
    yield torch.device("cuda:0")
    torch.cuda.synchronize()


def assert_close(got, ref, what=""):
    got = got.detach().to(torch.float64).cpu().numpy()
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    assert not bad.any(), f"{what}: max|err| {err.max():.3e}, {int(bad.sum())}/{bad.size} outside tolerance"


def single(d, dev, opt=None, ws=None):
    o = fd.fd_decode_fp8kv(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), d["k_scale"], d["v_scale"],
                           scale=d["scale"], opt=opt, ws=ws)
    torch.cuda.synchronize()
    return o


def paged(d, dev, opt=None, k_cache=None, v_cache=None, block_table=None):
    kc = (d["k_cache"] if k_cache is None else k_cache).to(dev)
    vc = (d["v_cache"] if v_cache is None else v_cache).to(dev)
    bt = (d["block_table"] if block_table is None else block_table).to(dev)
    o = fd.fd_paged_decode_fp8kv(d["q"].to(dev), kc, vc, bt, d["seq_lens"].to(dev), d["k_scale"], d["v_scale"],
                                 d["page_size"], scale=d["scale"], max_seq_len=d["max_seq_len"],
                                 total_kv=d["total_kv"], opt=opt)
    torch.cuda.synchronize()
    return o


def ref_single(d, heads=None):
    return oracle.decode_attention_e4m3(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["scale"],
                                        heads=heads)[0]


def ref_paged(d, pairs=None, k_cache=None, v_cache=None, block_table=None):
    return oracle.paged_decode_attention_e4m3(
        d["q"], d["k_cache"] if k_cache is None else k_cache, d["v_cache"] if v_cache is None else v_cache,
        d["block_table"] if block_table is None else block_table, d["seq_lens"], d["page_size"], d["k_scale"],
        d["v_scale"], d["scale"], pairs=pairs)[0]


# ------------------------------------------------------------------ decoding of the codes


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_every_code_decodes_exactly(dtype, kernel, device):
    """One key: o = v_scale * E4M3(v_0) exactly. The two KV heads' V rows hold all 256
    codes, so every code (including the two NaN codes, which give NaN) is converted once
    by each kernel; 4 query heads per KV head take the matrix-core kernel by default."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(2, 128)
    want = torch.from_numpy(oracle.dequantize_e4m3(codes.numpy(), 1 / 16)).to(DT[dtype])  # exact
    want = want.repeat_interleave(4, dim=0)
    d = inputs.with_fp8_kv(inputs.single_inputs(8, 2, 1, 128, dtype, 301), 1 / 16)
    d["v"] = codes[None].view(torch.float8_e4m3fn).contiguous()
    announce(f"every code single {dtype} {kernel}")
    o = single(d, device, opt=fd.options(kernel=kernel)).cpu()
    nan = torch.isnan(want)
    assert int(nan.sum()) == 8  # 0x7F and 0xFF, four query heads each
    assert torch.equal(torch.isnan(o), nan)
    assert torch.equal(o[~nan], want[~nan])
    # the same through a paged cache (page size 16, token 0 of page 2)
    p = inputs.with_fp8_kv(inputs.paged_inputs(1, 8, 2, 128, dtype, 16, [1], 302), 1 / 16)
    page = int(p["block_table"][0, 0])
    vc = p["v_cache"].view(torch.uint8).clone()
    vc[page, 0] = codes
    announce(f"every code paged {dtype} {kernel}")
    o = paged(p, device, opt=fd.options(kernel=kernel), v_cache=vc.view(torch.float8_e4m3fn))[0].cpu()
    assert torch.equal(torch.isnan(o), nan)
    assert torch.equal(o[~nan], want[~nan])


# ------------------------------------------------------------------ shapes, splits, kernels


@pytest.mark.parametrize("H,Hkv,kernel", [(32, 32, "auto"), (32, 4, "auto"), (32, 4, "valu"), (8, 8, "mfma"),
                                          (7, 1, "auto"), (64, 4, "mfma")])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_split_and_chunk_invariance(dtype, H, Hkv, kernel, device):
    """A 4099-token FP8 cache with peaked keys: every split count and chunk, either kernel."""
    d = inputs.with_fp8_kv(inputs.single_inputs(H, Hkv, 4099, 128, dtype, 310 + H + Hkv, peak_frac=0.01))
    ref = ref_single(d)
    for n, c in [(1, 0), (3, 0), (0, 0), (0, 64), (0, 1024)]:
        opt = fd.options(force_num_splits=n, force_chunk=c, kernel=kernel)
        plan = fd.decode_plan(H, Hkv, 4099, f"{dtype}_kv_e4m3", 0, opt)
        announce(f"invariance {dtype} H{H}/{Hkv} k{plan['kernel']} chunk {plan['chunk']}")
        assert_close(single(d, device, opt=opt), ref, f"H{H}/{Hkv} kernel {plan['kernel']} chunk {plan['chunk']}")


@pytest.mark.parametrize("H", [2, 4, 6, 12])
def test_mha_packed_kv_heads(H, device):
    """H = Hkv with 128-B E4M3 rows: 4 KV heads per workgroup when Hkv % 4 == 0, else 2."""
    d = inputs.with_fp8_kv(inputs.single_inputs(H, H, 1500, 128, "bf16", 360 + H))
    ref = ref_single(d)
    for opt in (None, fd.options(force_chunk=64)):
        plan = fd.decode_plan(H, H, 1500, "bf16_kv_e4m3", 0, opt)
        assert plan["kv_heads_per_group"] == (4 if H % 4 == 0 else 2)
        announce(f"mha packed H={H} hp={plan['kv_heads_per_group']} chunk {plan['chunk']}")
        assert_close(single(d, device, opt=opt), ref, f"H={H} chunk {plan['chunk']}")


@pytest.mark.parametrize("S", [0, 1, 17, 33, 65, 257, 1000])
def test_ragged_lengths(S, device):
    d = inputs.with_fp8_kv(inputs.single_inputs(8, 2, S, 128, "bf16", 320 + S))
    ref = ref_single(d)
    for opt in (None, fd.options(force_chunk=64), fd.options(kernel="valu", force_chunk=64)):
        announce(f"ragged S={S}")
        assert_close(single(d, device, opt=opt), ref, f"S={S}")


@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_uniform_codes_and_scales(kernel, device):
    """K and V codes uniform over all finite codes (every exponent, subnormals included),
    unequal scales k_scale = 2^-8, v_scale = 3."""
    rng = np.random.default_rng(330)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    d = inputs.single_inputs(16, 4, 2000, 128, "f16", 331)
    for key in ("k", "v"):
        d[key] = torch.from_numpy(rng.choice(finite, size=(2000, 4, 128))).view(torch.float8_e4m3fn)
    d["k_scale"], d["v_scale"] = 2.0 ** -8, 3.0
    announce(f"uniform codes {kernel}")
    o = single(d, device, opt=fd.options(kernel=kernel))
    ref = ref_single(d)
    assert_close(o, ref, f"uniform codes {kernel}")


# ------------------------------------------------------------------ workloads at full size


def test_workload_bf16_h32_s4096(device):
    """The 4k-token bf16 decode with its cache stored as E4M3 (scale 1/16)."""
    w = inputs.WORKLOADS["decode_bf16_h32_s4096"]
    d = inputs.with_fp8_kv(w.make())
    announce(w.name)
    assert_close(single(d, device), ref_single(d), w.name)


def test_workload_s131072(device):
    """The 128k-token peaked decode over an E4M3 cache, all 32 heads."""
    w = inputs.WORKLOADS["decode_bf16_h32_s131072_peaked"]
    d = inputs.with_fp8_kv(w.make())
    announce(w.name)
    assert_close(single(d, device), ref_single(d), w.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["paged_gqa4_bf16_b64_s1k-8k", "paged_gqa8_f16_b128_s256-64k"])
def test_paged_workload(name, device):
    """The GQA-4 (B = 64) and GQA-8 (B = 128, work list) paged batches with E4M3
    caches, every (sequence, head) row, both kernels."""
    w = inputs.WORKLOADS[name]
    announce(f"{w.name} (generating inputs)")
    d = inputs.with_fp8_kv(w.make())
    ref = ref_paged(d)
    for kernel in ("auto", "valu"):
        announce(f"{w.name} {kernel}")
        assert_close(paged(d, device, opt=fd.options(kernel=kernel)), ref, f"{w.name} {kernel}")


# ------------------------------------------------------------------ paged addressing


@pytest.mark.parametrize("kernel", ["auto", "valu"])
@pytest.mark.parametrize("ps", [1, 16, 128])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_paged_addressing_is_bit_exact(ps, dtype, kernel, device):
    """The same E4M3 tokens on in-order pages (identity table) and on shuffled pages:
    bit-identical outputs; NaN codes in tail slots and spare pages never reach o."""
    lens = [1, 17, 1000, 4096]
    B, H, Hkv = 4, 32, 8
    counts = [-(-L // ps) for L in lens]
    P = sum(counts)
    rng = np.random.default_rng(350 + ps)
    perm = rng.permutation(P)
    nan = torch.full((P + 3, ps, Hkv, 128), 0x7F, dtype=torch.uint8)
    kA, vA, kB, vB = nan.clone(), nan.clone(), nan.clone(), nan.clone()
    tA = torch.full((B, max(counts)), -1, dtype=torch.int32)
    tB = tA.clone()
    nxt = 0
    for b, L in enumerate(lens):
        kt = inputs.to_e4m3(inputs.normal(np.random.SeedSequence([351, b, 0]), (L, Hkv, 128), "f32"), 1 / 16)
        vt = inputs.to_e4m3(inputs.normal(np.random.SeedSequence([351, b, 1]), (L, Hkv, 128), "f32"), 1 / 16)
        kt, vt = kt.view(torch.uint8), vt.view(torch.uint8)
        for j in range(counts[b]):
            n = min(ps, L - j * ps)
            tA[b, j], tB[b, j] = nxt, int(perm[nxt])
            kA[nxt, :n], vA[nxt, :n] = kt[j * ps:j * ps + n], vt[j * ps:j * ps + n]
            kB[int(perm[nxt]), :n], vB[int(perm[nxt]), :n] = kt[j * ps:j * ps + n], vt[j * ps:j * ps + n]
            nxt += 1
    d = {"q": inputs.normal(np.random.SeedSequence(352), (B, H, 128), dtype), "seq_lens":
         torch.tensor(lens, dtype=torch.int32), "page_size": ps, "max_seq_len": max(lens), "total_kv": sum(lens),
         "scale": inputs.default_scale(128), "k_scale": 1 / 16, "v_scale": 1 / 16, "block_table": tA}
    outs = []
    for kc, vc, t in ((kA, vA, tA), (kB, vB, tB)):
        announce(f"paged bit-exact ps={ps} {dtype} {kernel}")
        outs.append(paged(d, device, opt=fd.options(force_chunk=512, kernel=kernel), k_cache=kc, v_cache=vc,
                          block_table=t).cpu())
    assert torch.isfinite(outs[0].float()).all()
    assert torch.equal(outs[0], outs[1])
    assert_close(outs[1], ref_paged(d, k_cache=kB, v_cache=vB, block_table=tB), f"paged ps={ps}")
