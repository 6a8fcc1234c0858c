"""The plain definition of single-query decode attention, in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page titles and sections):

* [FA] "FlashAttention 与推理算子" (anrans.github.io, ai-infra-handbooks):
  - section "标准注意力的问题": S = Q K^T / sqrt(d), P = softmax(S), O = P V.
    With one query row the scale is a parameter (the pages' callers pass
    1/sqrt(d) by default).
  - section "PagedAttention": token t of a sequence sits in physical page
    block_table[t / page_size], slot t % page_size.
  - section "decode 阶段的并行：Flash-Decoding 与 split-K": each KV segment
    yields its normalised output O_s and (m_s, l_s); they combine as
    m = max m_s, l = sum_s e^{m_s - m} l_s, O = sum_s e^{m_s - m} l_s O_s / l.
  - section "练习", exercise 2: a segment with no valid token (l = 0,
    m = -inf) is skipped.
  - section "一个分页 decode attention kernel（支持 GQA）": q head h reads KV
    head h / (num_heads / num_kv_heads); cache layout
    [num_pages, page_size, num_kv_heads, D]; q and out [num_seqs, num_heads, D].
* [FD] "[CUDA 优化实战] 纯手搓 flash decoding sm120" (wingedge777.com):
  - section "1. flash decoding": q [head, dim], k and v [seq, head, dim]; the
    KV sequence is cut into chunks of ``chunk`` tokens, ceil(S / chunk) of
    them, the last one shorter.
  - section "2. kernel 实现细节": each split stores its normalised output and a
    log-sum-exp; the merge takes the max lse, forms the global lse and sums
    the split outputs weighted by exp(lse_s - global lse).

Readings where the pages are silent: a sequence of length 0 gives o = 0 and
lse = -inf; log-sum-exp values are natural logarithms.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast of the stored input values to float64."""
    if hasattr(x, "detach"):  # torch tensor: bf16/f16/f32 -> f64 is exact
        import torch
        return x.detach().to(torch.float64).cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, H: int, Hkv: int) -> int:
    """GQA: consecutive groups of H / Hkv query heads share one KV head ([FA] paged GQA kernel)."""
    return h // (H // Hkv)


def scores(q_row: np.ndarray, keys: np.ndarray, scale: float) -> np.ndarray:
    """s_t = scale * q . k_t for every key row ([FA] "标准注意力的问题").

    ``q_row`` is one query [D] (result [L]) or several as columns [D, n]
    (result [L, n], column j the scores of query j)."""
    return (keys @ q_row) * np.float64(scale)


def softmax_weights(s: np.ndarray) -> np.ndarray:
    """P = softmax(s), materialised; the max is subtracted before exp (it cancels)."""
    e = np.exp(s - s.max())
    return e / e.sum()


def log_sum_exp(s: np.ndarray) -> float:
    """ln sum_t exp(s_t), natural log; -inf for an empty row."""
    if s.size == 0:
        return -np.inf
    m = s.max()
    return float(m + np.log(np.exp(s - m).sum()))


def weighted_sum(p: np.ndarray, values: np.ndarray) -> np.ndarray:
    """O = P V: one weight row [L] gives [D]; several rows [n, L] give [n, D]."""
    return p @ values


def decode_attention(q, k, v, scale: float, heads=None, return_weights: bool = False):
    """Single decode, contiguous KV.

    q [H, D], k and v [S, Hkv, D] (torch or numpy, any float dtype). Returns
    ``(o [n, D], lse [n])`` for the selected q heads (all by default), plus the
    list of weight rows if ``return_weights``.

    The heads are taken a KV head at a time: that head's keys and values are
    upcast exactly to float64 once, and the scores of all G query heads of the
    group are one matrix product (column j = query j); each column is then
    softmaxed on its own and P V is one more product. A group is always
    computed whole, whichever of its heads were asked for, so a head's result
    does not depend on the selection. Large caches are never copied whole.
    """
    H, D = q.shape
    S, Hkv = k.shape[0], k.shape[1]
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    o = np.zeros((len(heads), D), dtype=np.float64)
    lse = np.full(len(heads), -np.inf, dtype=np.float64)
    weights = [np.zeros(0)] * len(heads)
    groups: dict[int, list[int]] = {}
    for i, h in enumerate(heads):
        groups.setdefault(kv_head_of(h, H, Hkv), []).append(i)
    for g, idx in groups.items():
        if S == 0:
            continue
        members = [h for h in range(H) if kv_head_of(h, H, Hkv) == g]
        keys = _f64(k[:, g, :])
        values = _f64(v[:, g, :])
        q_cols = np.stack([_f64(q[h]) for h in members], axis=1)  # [D, G]
        s = scores(q_cols, keys, scale)                            # [S, G]
        p = np.stack([softmax_weights(s[:, j]) for j in range(len(members))])  # [G, S]
        og = weighted_sum(p, values)                               # [G, D]
        for i in idx:
            j = members.index(heads[i])
            o[i] = og[j]
            lse[i] = log_sum_exp(s[:, j])
            weights[i] = p[j]
    if return_weights:
        return o, lse, weights
    return o, lse


def _ints(x) -> np.ndarray:
    return np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int64)


def gather_pages(cache, table_row, L: int, page_size: int):
    """The first L token rows of one sequence in logical order ([FA] "PagedAttention").

    cache [num_pages, page_size, Hkv, D] (torch or numpy, stored dtype kept);
    table_row [max_blocks]. Token t is slot t % page_size of page
    table_row[t // page_size]. Returns [L, Hkv, D].
    """
    table_row = _ints(table_row)
    t = np.arange(int(L))
    page, slot = table_row[t // page_size], t % page_size
    if hasattr(cache, "detach"):
        import torch
        return cache[torch.from_numpy(page), torch.from_numpy(slot)]
    return np.asarray(cache)[page, slot]


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, page_size: int, scale: float,
                           pairs=None):
    """Batched paged GQA decode.

    q [B, H, D]; caches [num_pages, page_size, Hkv, D]; block_table [B, max_blocks];
    seq_lens [B]. ``pairs``: iterable of (b, h) to compute (all by default).
    Returns ``(o, lse)``: arrays [B, H, D] / [B, H] when ``pairs`` is None,
    else [n, D] / [n] in the order of ``pairs``.
    """
    table, lens = _ints(block_table), _ints(seq_lens)
    B, H, D = q.shape
    if pairs is None:
        o = np.zeros((B, H, D))
        lse = np.full((B, H), -np.inf)
        for b in range(B):
            kb = gather_pages(k_cache, table[b], lens[b], page_size)
            vb = gather_pages(v_cache, table[b], lens[b], page_size)
            o[b], lse[b] = decode_attention(q[b], kb, vb, scale)
        return o, lse
    pairs = [(int(b), int(h)) for b, h in pairs]
    o = np.zeros((len(pairs), D))
    lse = np.full(len(pairs), -np.inf)
    by_seq: dict[int, list[int]] = {}
    for i, (b, _) in enumerate(pairs):
        by_seq.setdefault(b, []).append(i)
    for b, idx in by_seq.items():  # one gather per sequence
        kb = gather_pages(k_cache, table[b], lens[b], page_size)
        vb = gather_pages(v_cache, table[b], lens[b], page_size)
        oo, ll = decode_attention(q[b], kb, vb, scale, heads=[pairs[i][1] for i in idx])
        o[idx], lse[idx] = oo, ll
    return o, lse


def split_bounds(L: int, chunk: int) -> list[tuple[int, int]]:
    """[start, end) of each KV split: ceil(L / chunk) splits, the last one shorter ([FD] §1)."""
    L, chunk = int(L), int(chunk)
    return [(s, min(s + chunk, L)) for s in range(0, L, chunk)]


def split_partials(q, k, v, scale: float, chunk: int, heads=None, bounds=None):
    """Per-split normalised outputs and natural-log lse ([FA] Flash-Decoding; [FD] §2).

    Each split's partial is the definition applied to that split's keys only.
    The splits are ``split_bounds(S, chunk)`` (the pages' cut), or the given
    ``bounds``: any list of [start, end) token ranges (the method is exact for
    every partition of the keys).
    Returns ``(O_s [n_heads, n_splits, D], lse_s [n_heads, n_splits])``.
    """
    H, D = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    if bounds is None:
        bounds = split_bounds(k.shape[0], chunk)
    O_s = np.zeros((len(heads), len(bounds), D))
    lse_s = np.full((len(heads), len(bounds)), -np.inf)
    for j, (a, b) in enumerate(bounds):
        O_s[:, j], lse_s[:, j] = decode_attention(q, k[a:b], v[a:b], scale, heads=heads)
    return O_s, lse_s


def paged_split_partials(q, k_cache, v_cache, block_table, seq_lens, page_size: int, scale: float,
                         chunk: int, b: int, h: int, bounds=None):
    """Split partials of one (sequence b, q head h) of a paged batch: ``(O_s [n, D], lse_s [n])``.

    The sequence's L_b tokens are gathered in logical order through its block
    table ([FA] "PagedAttention"), then cut as ``split_partials`` cuts a
    contiguous cache: ``split_bounds(L_b, chunk)``, or the given ``bounds``.
    """
    table, lens = _ints(block_table), _ints(seq_lens)
    kb = gather_pages(k_cache, table[b], lens[b], page_size)
    vb = gather_pages(v_cache, table[b], lens[b], page_size)
    O_s, lse_s = split_partials(q[b], kb, vb, scale, chunk, heads=[h], bounds=bounds)
    return O_s[0], lse_s[0]


def merge_lse(O_s, lse_s):
    """Merge one row's split partials by log-sum-exp ([FD] §2).

    O_s [n, D] normalised split outputs; lse_s [n] natural-log lse. A split
    with lse = -inf holds no valid token and is skipped ([FA] exercise 2).
    max_lse = max lse_s; global_lse = max_lse + ln sum exp(lse_s - max_lse);
    o = sum O_s exp(lse_s - global_lse). Returns ``(o [D], global_lse)``; with
    no valid split, o = 0 and lse = -inf.
    """
    O_s = np.asarray(O_s, dtype=np.float64)
    lse_s = np.asarray(lse_s, dtype=np.float64)
    keep = np.isfinite(lse_s)
    if not keep.any():
        return np.zeros(O_s.shape[-1]), -np.inf
    O_s, lse_s = O_s[keep], lse_s[keep]
    max_lse = lse_s.max()
    global_lse = max_lse + np.log(np.exp(lse_s - max_lse).sum())
    o = (O_s * np.exp(lse_s - global_lse)[:, None]).sum(axis=0)
    return o, float(global_lse)


def merge_m_l(O_s, m_s, l_s):
    """Merge one row's split partials from (m_s, l_s) ([FA] Flash-Decoding formula).

    m = max m_s; l = sum e^{m_s - m} l_s; O = sum e^{m_s - m} l_s O_s / l.
    Splits with l_s = 0 (m_s = -inf) are skipped ([FA] exercise 2).
    Returns ``(o [D], m, l)``; with no valid split, o = 0, m = -inf, l = 0.
    """
    O_s = np.asarray(O_s, dtype=np.float64)
    m_s = np.asarray(m_s, dtype=np.float64)
    l_s = np.asarray(l_s, dtype=np.float64)
    keep = l_s > 0
    if not keep.any():
        return np.zeros(O_s.shape[-1]), -np.inf, 0.0
    O_s, m_s, l_s = O_s[keep], m_s[keep], l_s[keep]
    m = m_s.max()
    w = np.exp(m_s - m) * l_s
    l = w.sum()
    o = (w[:, None] * O_s).sum(axis=0) / l
    return o, float(m), float(l)
