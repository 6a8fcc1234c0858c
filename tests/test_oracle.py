"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check uses the pages'
worked exercise, a closed form, a library routine (scipy, torch's CPU
attention), brute-force pure-Python recurrences, or an invariant. The last test
plants plausible mistakes in the oracle (on the CPU) and asserts that at least
one pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import oracle.decode as od
from oracle import loops

RNG = np.random.default_rng(12345)


def _unit(printed: str) -> float:
    """One unit in the last printed decimal place."""
    return 10.0 ** (-(len(printed.split(".")[1]) if "." in printed else 0))


def _close_to_printed(x: float, printed: str) -> bool:
    return abs(x - float(printed)) <= _unit(printed) + 1e-12


def _golden(name="worked_example.json"):
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", name), encoding="utf-8") as f:
        return json.load(f)


def _embed_scores(scores, values, D=1):
    """q = e_0 and k[t, 0] = s_t so that q . k_t = s_t; v[t, :] = value_t."""
    s = np.asarray(scores, dtype=np.float64)
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    k = np.zeros((len(s), 1, D))
    k[:, 0, 0] = s
    v = np.zeros((len(s), 1, D))
    v[:, 0, :] = np.asarray(values, dtype=np.float64)[:, None]
    return q, k, v


# ----------------------------------------------------------------------------- pins


def pin_worked_example() -> bool:
    g = _golden()
    trace = []
    final = loops.online_from_scores(g["scores"], g["values"], trace)
    ok = _close_to_printed(final, g["final"])
    for got, want in zip(trace, g["after_block"]):
        ok &= _close_to_printed(got["m"], want["m"])
        ok &= _close_to_printed(got["l"], want["l"])
        ok &= _close_to_printed(got["O"], want["O"])
        ok &= all(_close_to_printed(a, b) for a, b in zip(got["p"], want["p"]))
        if "correction" in want:
            ok &= _close_to_printed(got["correction"], want["correction"])
    flat_s = [x for blk in g["scores"] for x in blk]
    flat_v = [x for blk in g["values"] for x in blk]
    for D in (1, 4, 128):
        q, k, v = _embed_scores(flat_s, flat_v, D)
        o, lse, w = oracle.decode_attention(q, k, v, 1.0, return_weights=True)
        ok &= _close_to_printed(float(o[0, 0]), g["final"])
        ok &= bool(np.all(o[0] == o[0, 0]))
        # the page's direct computation: weights e^{s_t} summing to 178.6
        total = float(np.exp(lse[0]))
        ok &= _close_to_printed(total, g["direct_weight_sum"])
        ok &= all(_close_to_printed(float(w[0][t] * total), g["direct_weights"][t]) for t in range(4))
        ok &= all(_close_to_printed(float(w[0][t] * total * flat_v[t]), g["direct_weighted_terms"][t])
                  for t in range(4))
    return bool(ok)


def pin_two_keys_logistic() -> bool:
    """S = 2: o = expit(s0 - s1) v0 + expit(s1 - s0) v1, s_t = scale q . k_t."""
    ok = True
    rng = np.random.default_rng(7)
    for scale in (0.37, 1.0, 2.5):
        q = rng.standard_normal((1, 8))
        k = rng.standard_normal((2, 1, 8))
        v = rng.standard_normal((2, 1, 8))
        s0 = scale * sum(q[0, d] * k[0, 0, d] for d in range(8))
        s1 = scale * sum(q[0, d] * k[1, 0, d] for d in range(8))
        want = scipy.special.expit(s0 - s1) * v[0, 0] + scipy.special.expit(s1 - s0) * v[1, 0]
        o, lse = oracle.decode_attention(q, k, v, scale)
        ok &= np.allclose(o[0], want, rtol=1e-12, atol=1e-13)
        ok &= abs(lse[0] - np.logaddexp(s0, s1)) < 1e-12
    return bool(ok)


def pin_rows_sum_to_one() -> bool:
    q = RNG.standard_normal((4, 16))
    k = RNG.standard_normal((300, 2, 16)) * 3
    v = RNG.standard_normal((300, 2, 16))
    _, _, w = oracle.decode_attention(q, k, v, 0.25, return_weights=True)
    return all(abs(p.sum() - 1.0) <= 1e-12 and p.min() >= 0 for p in w)


def pin_identical_keys_mean() -> bool:
    q = RNG.standard_normal((2, 8))
    k = np.repeat(RNG.standard_normal((1, 1, 8)), 37, axis=0)
    v = RNG.standard_normal((37, 1, 8))
    o, lse = oracle.decode_attention(q, k, v, 0.5)
    ok = np.allclose(o, v[:, 0, :].mean(axis=0)[None, :].repeat(2, 0), rtol=1e-12, atol=1e-13)
    s = 0.5 * (q @ k[0, 0])
    ok &= np.allclose(lse, s + math.log(37), rtol=1e-12)
    return bool(ok)


def pin_zero_scale_mean() -> bool:
    q = RNG.standard_normal((3, 8))
    k = RNG.standard_normal((50, 3, 8))
    v = RNG.standard_normal((50, 3, 8))
    o, lse = oracle.decode_attention(q, k, v, 0.0)
    ok = np.allclose(o, v.mean(axis=0), rtol=1e-12, atol=1e-13)
    ok &= np.allclose(lse, math.log(50), rtol=1e-12)
    return bool(ok)


def pin_single_key_exact() -> bool:
    gen = torch.Generator().manual_seed(11)
    q = torch.randn(4, 128, generator=gen).to(torch.bfloat16)
    k = torch.randn(1, 4, 128, generator=gen).to(torch.bfloat16)
    v = torch.randn(1, 4, 128, generator=gen).to(torch.bfloat16)
    o, _ = oracle.decode_attention(q, k, v, 0.088388)
    return bool(np.array_equal(o, v[0].to(torch.float64).numpy()))


def pin_lse_scipy() -> bool:
    q = RNG.standard_normal((3, 32))
    k = RNG.standard_normal((200, 3, 32)) * 2
    v = RNG.standard_normal((200, 3, 32))
    _, lse = oracle.decode_attention(q, k, v, 0.3)
    want = [scipy.special.logsumexp(0.3 * (k[:, h, :] @ q[h])) for h in range(3)]
    return bool(np.allclose(lse, want, rtol=1e-13, atol=1e-13))


def pin_torch_sdpa() -> bool:
    """torch's CPU scaled_dot_product_attention in float64, with its own GQA grouping."""
    ok = True
    for H, Hkv, S, D in ((8, 2, 300, 128), (4, 4, 33, 64), (6, 3, 1, 16)):
        q = RNG.standard_normal((H, D))
        k = RNG.standard_normal((S, Hkv, D))
        v = RNG.standard_normal((S, Hkv, D))
        scale = 1.0 / math.sqrt(D)
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
        tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale, enable_gqa=True)
        o, _ = oracle.decode_attention(q, k, v, scale)
        ok &= np.allclose(o, ref[0, :, 0, :].numpy(), rtol=1e-11, atol=1e-12)
    return bool(ok)


def pin_gqa_mapping() -> bool:
    """Plant one dominant key per KV head: q head h must return that key's value
    for KV head h // (H / Hkv) (consecutive q heads share a KV head)."""
    H, Hkv, S, D = 8, 4, 20, 16
    q = np.zeros((H, D))
    q[:, 0] = 1.0
    k = np.zeros((S, Hkv, D))
    v = RNG.standard_normal((S, Hkv, D))
    hot = [3, 11, 5, 17]
    for g, t in enumerate(hot):
        k[t, g, 0] = 60.0  # e^-60 leaves every other weight below 1e-26
    o, _ = oracle.decode_attention(q, k, v, 1.0)
    want = np.stack([v[hot[h // 2], h // 2] for h in range(H)])
    return bool(np.allclose(o, want, rtol=1e-12, atol=1e-20))


def pin_brute_force_recurrences() -> bool:
    """Pure-Python three-pass == pure-Python online (several block sizes) == oracle, tiny inputs."""
    rng = np.random.default_rng(99)
    ok = True
    for trial in range(60):
        S = int(rng.integers(1, 9))
        D = int(rng.integers(1, 5))
        scale = float(rng.uniform(0.1, 3.0))
        q = rng.standard_normal(D)
        keys = rng.standard_normal((S, D)) * rng.uniform(0.5, 4)
        vals = rng.standard_normal((S, D))
        o3, l3 = loops.three_pass(q.tolist(), keys.tolist(), vals.tolist(), scale)
        o_np, l_np = oracle.decode_attention(q[None], keys[:, None, :], vals[:, None, :], scale)
        ok &= np.allclose(o3, o_np[0], rtol=1e-12, atol=1e-13) and abs(l3 - l_np[0]) < 1e-12
        for block in (1, 2, 3, S):
            oo, lo = loops.online(q.tolist(), keys.tolist(), vals.tolist(), scale, block)
            ok &= np.allclose(oo, o3, rtol=1e-12, atol=1e-13) and abs(lo - l3) < 1e-12
    return bool(ok)


def pin_split_invariance() -> bool:
    """merge(partials) == full attention for chunks that do and do not divide S, and for
    explicit partitions with unequal ranges (a long last range, a one-token range)."""
    H, Hkv, S, D = 4, 2, 1001, 32
    q = RNG.standard_normal((H, D))
    k = RNG.standard_normal((S, Hkv, D)) * 2
    v = RNG.standard_normal((S, Hkv, D))
    o_full, lse_full = oracle.decode_attention(q, k, v, 0.2)
    ok = True
    cases = [(chunk, None) for chunk in (1, 7, 16, 64, 1000, S, 4096)]
    cases += [(0, [(0, 64), (64, 128), (128, S)]), (0, [(0, 1), (1, 500), (500, S)])]
    for chunk, bounds in cases:
        O_s, lse_s = oracle.split_partials(q, k, v, 0.2, chunk, bounds=bounds)
        ok &= O_s.shape[1] == (-(-S // chunk) if bounds is None else len(bounds))
        for h in range(H):
            o, lse = oracle.merge_lse(O_s[h], lse_s[h])
            ok &= np.allclose(o, o_full[h], rtol=1e-12, atol=1e-13)
            ok &= abs(lse - lse_full[h]) < 1e-11
            ok &= abs(scipy.special.logsumexp(lse_s[h]) - lse_full[h]) < 1e-11
    return bool(ok)


def pin_merge_forms_agree() -> bool:
    """The lse merge and the (m, l) merge agree (lse_s = m_s + ln l_s); empty splits are skipped."""
    rng = np.random.default_rng(5)
    ok = True
    for n in (1, 2, 5, 9):
        O_s = rng.standard_normal((n, 16))
        m_s = rng.uniform(-5, 5, n)
        l_s = rng.uniform(0.5, 30, n)
        if n > 2:
            m_s[1], l_s[1] = -np.inf, 0.0
            O_s[1] = np.nan  # must never be read
        lse_s = np.where(l_s > 0, m_s + np.log(np.where(l_s > 0, l_s, 1)), -np.inf)
        o1, lse = oracle.merge_lse(O_s, lse_s)
        o2, m, l = oracle.merge_m_l(O_s, m_s, l_s)
        ok &= np.allclose(o1, o2, rtol=1e-12, atol=1e-13) and np.isfinite(o1).all()
        ok &= abs(lse - (m + math.log(l))) < 1e-12
    o, lse = oracle.merge_lse(np.full((3, 4), np.nan), np.full(3, -np.inf))
    ok &= np.array_equal(o, np.zeros(4)) and lse == -np.inf
    return bool(ok)


def _paged_case(lens, H=32, Hkv=8, D=16, ps=16, seed=3):
    """A pool built by hand from contiguous per-sequence K/V, pages placed by a shuffle."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    q = rng.standard_normal((B, H, D))
    ks = [rng.standard_normal((L, Hkv, D)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)) for L in lens]
    counts = [-(-L // ps) for L in lens]
    P = sum(counts)
    perm = rng.permutation(P)
    kc = np.full((P + 3, ps, Hkv, D), np.nan)  # 3 unreferenced pages, NaN everywhere unused
    vc = np.full((P + 3, ps, Hkv, D), np.nan)
    table = np.full((B, max(counts + [1])), -1, dtype=np.int64)
    nxt = 0
    for b, L in enumerate(lens):
        for j in range(counts[b]):
            page = perm[nxt]
            nxt += 1
            table[b, j] = page
            for slot in range(ps):
                t = j * ps + slot
                if t < L:
                    kc[page, slot] = ks[b][t]
                    vc[page, slot] = vs[b][t]
    return q, ks, vs, kc, vc, table, np.asarray(lens)


def pin_paged_equals_contiguous() -> bool:
    """Lengths of the pages' paged harness (1, 17, 1000, 4096) over a shuffled pool whose
    unused slots and pages hold NaN: the paged oracle equals the contiguous one exactly."""
    lens = [1, 17, 1000, 4096]
    q, ks, vs, kc, vc, table, L = _paged_case(lens)
    o, lse = oracle.paged_decode_attention(q, kc, vc, table, L, 16, 0.25)
    ok = np.isfinite(o).all()
    for b in range(len(lens)):
        ob, lb = oracle.decode_attention(q[b], ks[b], vs[b], 0.25)
        ok &= np.array_equal(o[b], ob) and np.array_equal(lse[b], lb)
    pairs = [(3, 31), (0, 0), (2, 9)]
    op, lp = oracle.paged_decode_attention(q, kc, vc, table, L, 16, 0.25, pairs=pairs)
    ok &= all(np.array_equal(op[i], o[b, h]) for i, (b, h) in enumerate(pairs))
    return bool(ok)


def pin_paged_split_partials() -> bool:
    """Split partials of a paged sequence equal the contiguous split partials of the same
    tokens (pinned by pin_split_invariance) for the pages' cut and for the library's
    (max(1, L // chunk) splits, the last one taking the remainder). The pool is built by
    hand with NaN in every unused slot and page, so a wrong page, slot, sequence or
    length shows. The split lse values combine (scipy logsumexp) to the lse of the whole
    sequence, and merge_lse of the partials gives the paged result."""
    lens = [1, 17, 1000, 4096]
    q, ks, vs, kc, vc, table, L = _paged_case(lens)
    o_full, lse_full = oracle.paged_decode_attention(q, kc, vc, table, L, 16, 0.25)
    ok = True
    for b, h, chunk, library_cut in ((0, 0, 16, False), (1, 7, 16, True), (2, 9, 64, False), (2, 30, 64, True),
                                     (3, 31, 1024, True), (3, 4, 100, False), (3, 12, 4096, True)):
        n = max(1, lens[b] // chunk)
        bounds = ([(s * chunk, lens[b] if s == n - 1 else (s + 1) * chunk) for s in range(n)]
                  if library_cut else None)
        O_s, lse_s = oracle.paged_split_partials(q, kc, vc, table, L, 16, 0.25, chunk, b, h, bounds=bounds)
        Oc, lc = oracle.split_partials(q[b], ks[b], vs[b], 0.25, chunk, heads=[h], bounds=bounds)
        ok &= O_s.shape == Oc[0].shape and np.array_equal(O_s, Oc[0]) and np.array_equal(lse_s, lc[0])
        ok &= bool(np.isfinite(O_s).all()) and O_s.shape[0] == (n if library_cut else -(-lens[b] // chunk))
        ok &= abs(scipy.special.logsumexp(lse_s) - lse_full[b, h]) < 1e-11
        o, _ = oracle.merge_lse(O_s, lse_s)
        ok &= np.allclose(o, o_full[b, h], rtol=1e-12, atol=1e-13)
    return bool(ok)


def pin_e4m3_decoding() -> bool:
    """Every E4M3 code against torch's float8_e4m3fn decoding (a library routine), plus
    the format's landmarks: 1.0, the largest finite 448, the smallest subnormal 2^-9."""
    import torch
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    table = oracle.dequantize_e4m3(np.arange(256, dtype=np.uint8), 1.0)
    ok = np.array_equal(np.isnan(lib), np.isnan(table))
    ok &= np.array_equal(lib[~np.isnan(lib)], table[~np.isnan(table)])
    ok &= table[0x38] == 1.0 and table[0x7E] == 448.0 and table[0x01] == 2.0 ** -9 and table[0xB8] == -1.0
    ok &= np.array_equal(oracle.dequantize_e4m3(np.array([0x38, 0x40], dtype=np.uint8), 0.0625), [0.0625, 0.125])
    return bool(ok)


def pin_e4m3_attention() -> bool:
    """FP8 attention == the plain definition on the same values written out by hand: K
    holds k_scale * {0, 1, 2, 3}, V holds v_scale * {-1, 1.5, 448} (all exact E4M3 values;
    codes by torch's float8 encoder), with k_scale != v_scale; and the paged form over a
    shuffled two-page table equals the contiguous one."""
    import torch
    ks, vs = 0.25, 3.0
    kvals = np.array([[0.0, 1.0], [2.0, 3.0], [1.0, 0.0]])          # [S=3, D=2]
    vvals = np.array([[-1.0, 1.5], [448.0, -1.0], [1.5, 1.5]])
    codes = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q = np.array([[0.5, -1.0], [2.0, 0.25]])
    o, lse = oracle.decode_attention_e4m3(q, codes(kvals)[:, None], codes(vvals)[:, None], ks, vs, 0.7)
    s = 0.7 * (q @ (ks * kvals).T)                                  # [H, S], written out
    w = np.exp(s - s.max(axis=1, keepdims=True))
    want = (w / w.sum(axis=1, keepdims=True)) @ (vs * vvals)
    ok = np.allclose(o, want, rtol=1e-13, atol=0) and np.allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-13)
    kc = np.zeros((2, 2, 1, 2), np.uint8)
    vc = np.zeros((2, 2, 1, 2), np.uint8)
    kc[1, 0, 0], kc[1, 1, 0], kc[0, 0, 0] = codes(kvals)
    vc[1, 0, 0], vc[1, 1, 0], vc[0, 0, 0] = codes(vvals)
    po, plse = oracle.paged_decode_attention_e4m3(q[None], kc, vc, np.array([[1, 0]]), np.array([3]), 2, ks, vs,
                                                  0.7)
    ok &= np.allclose(po[0], want, rtol=1e-13, atol=0)
    po2, _ = oracle.paged_decode_attention_e4m3(q[None], kc, vc, np.array([[1, 0]]), np.array([3]), 2, ks, vs, 0.7,
                                                pairs=[(0, 1)])
    ok &= np.allclose(po2[0], want[1], rtol=1e-13, atol=0)
    return bool(ok)


def pin_prefill_torch_sdpa() -> bool:
    """Prefill against torch's CPU scaled_dot_product_attention in float64 (is_causal and
    not), with its own GQA grouping, at N not a multiple of any tile."""
    ok = True
    for B, N, H, Hkv, D, causal in ((2, 37, 4, 2, 16, True), (1, 50, 3, 3, 8, False), (1, 1, 2, 1, 4, True)):
        q = RNG.standard_normal((B, N, H, D))
        k = RNG.standard_normal((B, N, Hkv, D))
        v = RNG.standard_normal((B, N, Hkv, D))
        tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3, is_causal=causal,
                                                               enable_gqa=True)
        o, _ = oracle.prefill_attention(q, k, v, 0.3, causal)
        ok &= np.allclose(o, ref.numpy().transpose(0, 2, 1, 3), rtol=1e-11, atol=1e-12)
    return bool(ok)


def pin_prefill_rows_are_decodes() -> bool:
    """Causal row i is the decode of query i over keys 0..i (its lse too); row 0 returns
    v_0 exactly; identical keys give the running mean of V; non-causal rows see all keys."""
    B, N, H, Hkv, D = 1, 23, 4, 2, 8
    q = RNG.standard_normal((B, N, H, D))
    k = RNG.standard_normal((B, N, Hkv, D))
    v = RNG.standard_normal((B, N, Hkv, D))
    o, lse = oracle.prefill_attention(q, k, v, 0.7, True)
    ok = True
    for i in (0, 1, 7, 22):
        od, ld = oracle.decode_attention(q[0, i], k[0, :i + 1], v[0, :i + 1], 0.7)
        ok &= np.allclose(o[0, i], od, rtol=1e-12, atol=1e-13) and np.allclose(lse[0, i], ld, rtol=1e-12)
    ok &= np.array_equal(o[0, 0], np.repeat(v[0, 0], 2, axis=0))
    on, _ = oracle.prefill_attention(q, k, v, 0.7, False)
    od, _ = oracle.decode_attention(q[0, 5], k[0], v[0], 0.7)
    ok &= np.allclose(on[0, 5], od, rtol=1e-12, atol=1e-13)
    kk = np.repeat(k[:, :1], N, axis=1)
    oi, _ = oracle.prefill_attention(q, kk, v, 0.7, True)
    means = np.cumsum(v[0], axis=0) / np.arange(1, N + 1)[:, None, None]
    ok &= np.allclose(oi[0], np.repeat(means, 2, axis=1), rtol=1e-12, atol=1e-13)
    return bool(ok)


PINS = [pin_worked_example, pin_two_keys_logistic, pin_rows_sum_to_one, pin_identical_keys_mean,
        pin_zero_scale_mean, pin_single_key_exact, pin_lse_scipy, pin_torch_sdpa, pin_gqa_mapping,
        pin_brute_force_recurrences, pin_split_invariance, pin_merge_forms_agree,
        pin_paged_equals_contiguous, pin_paged_split_partials, pin_e4m3_decoding, pin_e4m3_attention, pin_prefill_torch_sdpa,
        pin_prefill_rows_are_decodes]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin()


def test_empty_sequence_reading():
    """Reading adopted where the pages are silent: L = 0 gives o = 0, lse = -inf."""
    q = np.ones((2, 8))
    k = np.zeros((0, 1, 8))
    o, lse = oracle.decode_attention(q, k, k, 1.0)
    assert np.array_equal(o, np.zeros((2, 8))) and np.all(lse == -np.inf)
    o, lse = oracle.paged_decode_attention(q[None], np.zeros((1, 16, 1, 8)), np.zeros((1, 16, 1, 8)),
                                           np.array([[-1]]), np.array([0]), 16, 1.0)
    assert np.array_equal(o, np.zeros((1, 2, 8)))


def test_split_bounds_cover_every_token_once():
    for L in (0, 1, 63, 64, 65, 131073):
        for chunk in (1, 64, 2048):
            b = oracle.split_bounds(L, chunk)
            assert len(b) == -(-L // chunk)
            covered = [t for s, e in b for t in range(s, e)] if L < 5000 else None
            if covered is not None:
                assert covered == list(range(L))
            assert all(e - s == chunk for s, e in b[:-1]) and (not b or b[-1][1] == L)


# ----------------------------------------------------------------------- planted mistakes

MUTANTS = {
    "gqa_mapping_modulo": ("kv_head_of", lambda h, H, Hkv: h % Hkv),
    "scale_dropped": ("scores", lambda q_row, keys, scale: keys @ q_row),
    "score_sign": ("scores", lambda q_row, keys, scale: -(keys @ q_row) * scale),
    "softmax_unnormalised": ("softmax_weights", lambda s: np.exp(s - s.max())),
    "softmax_no_exp": ("softmax_weights", lambda s: (s - s.min()) / (s - s.min()).sum()),
    "values_token_reversed": ("weighted_sum", lambda p, values: p @ values[::-1]),
    "lse_missing_max": ("log_sum_exp", lambda s: float(np.log(np.exp(s - s.max()).sum()))),
    "split_floor_drops_tail": ("split_bounds",
                               lambda L, chunk: [(s, s + chunk) for s in range(0, (L // chunk) * chunk, chunk)]),
    "merge_ignores_lse": ("merge_lse", lambda O_s, lse_s: (np.asarray(O_s).mean(axis=0), float(np.max(lse_s)))),
    "page_slot_swapped": ("gather_pages", None),
    "paged_partials_ignore_bounds": ("paged_split_partials", lambda *a, bounds=None: _bad_partials(*a, cut="pages")),
    "paged_partials_drop_last_token": ("paged_split_partials", lambda *a, bounds=None: _bad_partials(*a, bounds=bounds,
                                                                                                    short=1)),
    "e4m3_bias_8": ("E4M3_TABLE", None),
    "e4m3_scales_swapped": ("decode_attention_e4m3", None),
    "causal_off_by_one": ("causal_mask", lambda n_q, n_k: np.arange(n_k)[None, :] < np.arange(n_q)[:, None]),
    "causal_transposed": ("causal_mask", lambda n_q, n_k: np.arange(n_k)[None, :] >= np.arange(n_q)[:, None]),
}


def _bad_gather(cache, table_row, L, page_size):
    """Slots read back to front inside each page."""
    table_row = np.asarray(table_row, dtype=np.int64)
    t = np.arange(int(L))
    return np.asarray(cache)[table_row[t // page_size], (page_size - 1) - t % page_size]


def _bad_partials(q, k_cache, v_cache, block_table, seq_lens, page_size, scale, chunk, b, h, bounds=None,
                  cut="given", short=0):
    """paged_split_partials with a planted mistake: the given token ranges ignored (the
    pages' cut used instead), or a sequence gathered one token short."""
    table, lens = od._ints(block_table), od._ints(seq_lens)
    kb = od.gather_pages(k_cache, table[b], lens[b] - short, page_size)
    vb = od.gather_pages(v_cache, table[b], lens[b] - short, page_size)
    O_s, lse_s = od.split_partials(q[b], kb, vb, scale, chunk, heads=[h], bounds=None if cut == "pages" else bounds)
    return O_s[0], lse_s[0]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if attr == "E4M3_TABLE":
        import oracle.fp8 as of
        bad = np.array([of.e4m3_value(c) / 2.0 for c in range(256)])  # exponent bias 8
        monkeypatch.setattr(of, "E4M3_TABLE", bad)
    elif attr == "decode_attention_e4m3":
        import oracle.fp8 as of
        good = of.dequantize_e4m3

        def swapped(codes, scale):  # K gets v_scale and V gets k_scale
            return good(codes, {0.25: 3.0, 3.0: 0.25}.get(scale, scale))
        monkeypatch.setattr(of, "dequantize_e4m3", swapped)
    elif attr == "causal_mask":
        import oracle.prefill as opf
        monkeypatch.setattr(opf, "causal_mask", fn)
    else:
        if fn is None:
            fn = _bad_gather
        monkeypatch.setattr(od, attr, fn)
        monkeypatch.setattr(oracle, attr, fn, raising=False)
    results = {}
    for pin in PINS:
        try:
            results[pin.__name__] = pin()
        except Exception:  # a crash also counts as caught
            results[pin.__name__] = False
    assert not all(results.values()), f"mutant {name} passed every pin"
