"""Prefill (many-query) attention with an optional causal mask, in numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "FlashAttention 与推理算子" (anrans.github.io, ai-infra-handbooks):
  - section "标准注意力的问题": S = Q K^T / sqrt(d), P = softmax(S), O = P V;
  - section "FlashAttention：分块 + online softmax", paragraph on the causal mask
    of decoder self-attention: query i sees keys 0 .. i only;
  - section "推理：prefill 与 decode": prefill runs this over the whole prompt.
The scale is a parameter (1/sqrt(d) by default at the callers). GQA maps query
head h to KV head h // (H / Hkv), as for decode.

Layouts (token-major, the decode cache layout per sequence):
  q, o [B, N, H, D];  k, v [B, N, Hkv, D].
The plain definition is written per (sequence, head): the N x N score matrix,
the mask, a row softmax (the row max subtracted before exp), then P V.
"""
from __future__ import annotations

import numpy as np

from .decode import _f64, kv_head_of


def causal_mask(n_q: int, n_k: int) -> np.ndarray:
    """Boolean [n_q, n_k], True where key j is visible to query i (j <= i)."""
    return np.arange(n_k)[None, :] <= np.arange(n_q)[:, None]


def head_attention(q_h, k_g, v_g, scale: float, causal: bool):
    """One (sequence, head): q_h [N, D], k_g and v_g [N, D] in float64.
    Returns (o [N, D], lse [N]); lse is the natural-log sum of exp(scores)."""
    s = (q_h @ k_g.T) * np.float64(scale)
    if causal:
        s = np.where(causal_mask(s.shape[0], s.shape[1]), s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l_sum = e.sum(axis=1, keepdims=True)
    return (e / l_sum) @ v_g, (m + np.log(l_sum))[:, 0]


def prefill_attention(q, k, v, scale: float, causal: bool, heads=None, batches=None):
    """Attention of every query row over the keys it may see.

    q [B, N, H, D], k and v [B, N, Hkv, D] (torch or numpy; upcast exactly to
    float64 one (sequence, KV head) at a time). ``heads`` / ``batches`` select
    what to compute (all by default). Returns ``(o, lse)``: o [nb, N, nh, D],
    lse [nb, N, nh].
    """
    B, N, H, D = q.shape
    Hkv = k.shape[2]
    heads = list(range(H)) if heads is None else [int(h) for h in heads]
    batches = list(range(B)) if batches is None else [int(b) for b in batches]
    o = np.zeros((len(batches), N, len(heads), D))
    lse = np.zeros((len(batches), N, len(heads)))
    for i, b in enumerate(batches):
        cache = {}
        for j, h in enumerate(heads):
            g = kv_head_of(h, H, Hkv)
            if g not in cache:
                cache = {g: (_f64(k[b, :, g, :]), _f64(v[b, :, g, :]))}
            kg, vg = cache[g]
            o[i, :, j], lse[i, :, j] = head_attention(_f64(q[b, :, h, :]), kg, vg, scale, causal)
    return o, lse
