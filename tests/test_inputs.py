"""The seeded generators: determinism, shapes, dtype rounding and page bookkeeping."""
import numpy as np
import torch

from decode_attention_13_amd import inputs


def test_normal_is_deterministic_and_thread_independent(monkeypatch):
    ss = np.random.SeedSequence(77)
    a = inputs.normal(ss, (3, inputs.CHUNK_ELEMS // 2 + 5), "bf16")
    monkeypatch.setattr(inputs, "_workers", lambda: 1)
    b = inputs.normal(ss, (3, inputs.CHUNK_ELEMS // 2 + 5), "bf16")
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    c = inputs.normal(np.random.SeedSequence(78), (3, inputs.CHUNK_ELEMS // 2 + 5), "bf16")
    assert not torch.equal(a, c)


def test_normal_rounds_float32_draws_to_nearest_even():
    ss = np.random.SeedSequence(5)
    x16 = inputs.normal(ss, (1000,), "f16")
    x32 = inputs.normal(ss, (1000,), "f32")
    assert torch.equal(x16, x32.to(torch.float16))
    assert abs(float(x32.mean())) < 0.15 and 0.85 < float(x32.std()) < 1.15


def test_single_inputs_peaked_rows():
    d = inputs.single_inputs(4, 2, 1000, 16, "bf16", 9, peak_frac=0.01)
    plain = inputs.single_inputs(4, 2, 1000, 16, "bf16", 9)
    rows = d["peak_rows"]
    assert len(rows) == 10 and len(set(rows.tolist())) == 10
    assert torch.equal(d["k"][rows], plain["k"][rows] * 8)
    mask = torch.ones(1000, dtype=torch.bool)
    mask[torch.from_numpy(rows)] = False
    assert torch.equal(d["k"][mask], plain["k"][mask])
    assert torch.equal(d["v"], plain["v"]) and torch.equal(d["q"], plain["q"])


def test_page_table_uses_every_page_once():
    lens = [1, 17, 1000, 4096, 16, 0]
    table, P, mb = inputs.page_table(lens, 16, 7)
    counts = [-(-L // 16) for L in lens]
    assert P == sum(counts) and mb == max(counts)
    used = []
    for b, c in enumerate(counts):
        assert (table[b, c:] == -1).all()
        used += table[b, :c].tolist()
    assert sorted(used) == list(range(P))
    ident, _, _ = inputs.page_table(lens, 16, None)
    assert sorted(ident[ident >= 0].tolist()) == list(range(P))
    assert ident[3, 0] == sum(counts[:3])


def test_workload_lengths():
    w4 = inputs.WORKLOADS["paged_gqa4_bf16_b64_s1k-8k"]
    L4 = w4.seq_lens()
    assert len(L4) == 64 and L4.min() >= 1024 and L4.max() <= 8192
    w5 = inputs.WORKLOADS["paged_gqa8_f16_b128_s256-64k"]
    L5 = w5.seq_lens()
    assert len(L5) == 128 and L5.min() >= 256 and L5.max() <= 65536
    assert np.array_equal(L5, w5.seq_lens())
    assert inputs.WORKLOADS["decode_bf16_h32_s4096"].kv_bytes() == 67108864
    assert inputs.WORKLOADS["decode_f32_h8_s512"].kv_bytes() == 4194304


def test_default_scale_is_float32():
    s = inputs.default_scale(128)
    assert s == float(np.float32(1 / np.sqrt(128)))
