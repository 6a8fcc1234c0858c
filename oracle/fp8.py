"""FP8 E4M3 KV-cache values, in float64. TEST INFRASTRUCTURE ONLY (see the package docstring).

"FlashAttention 与推理算子", in its list of improvements after the paged GQA
kernel, notes that a real KV cache is BF16 or FP8, read with 128-bit loads
and converted to FP32 in registers. The pages fix no quantisation scheme; the
reading here is the plainest one: every K and V element is an OCP FP8 E4M3
code (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
subnormal; S.1111.111 is NaN; no infinities; largest finite value 448), and the
cached value is code value x a per-tensor scale (k_scale for K, v_scale for
V). Attention is then the plain definition over these values.
"""
from __future__ import annotations

import math

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    mant = code & 0x7
    if exp == 0xF and mant == 0x7:
        return math.nan
    if exp == 0:
        return sign * (mant / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + mant / 8.0) * 2.0 ** (exp - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def dequantize_e4m3(codes, scale: float) -> np.ndarray:
    """Cached values of E4M3 codes (a uint8 array or a torch float8_e4m3fn tensor) times scale."""
    if hasattr(codes, "detach"):
        import torch
        codes = codes.detach().cpu().contiguous().view(torch.uint8).numpy()
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * np.float64(scale)


def decode_attention_e4m3(q, k_codes, v_codes, k_scale: float, v_scale: float, scale: float, heads=None):
    """Plain decode attention over the values an E4M3 cache holds: K = k_scale * E4M3(k_codes),
    V = v_scale * E4M3(v_codes); q is kept in its own precision. Returns ``(o, lse)``."""
    from .decode import decode_attention
    return decode_attention(q, dequantize_e4m3(k_codes, k_scale), dequantize_e4m3(v_codes, v_scale), scale,
                            heads=heads)


def paged_decode_attention_e4m3(q, k_cache, v_cache, block_table, seq_lens, page_size: int, k_scale: float,
                                v_scale: float, scale: float, pairs=None):
    """Batched paged GQA decode over E4M3 caches: each sequence's code rows are gathered
    through its block table, dequantised, and fed to the plain definition.

    Arguments and results as ``paged_decode_attention``, plus the two scales.
    """
    from .decode import _ints, decode_attention, gather_pages
    table, lens = _ints(block_table), _ints(seq_lens)
    B, H, D = q.shape

    def rows(b):
        kb = gather_pages(k_cache, table[b], lens[b], page_size)
        vb = gather_pages(v_cache, table[b], lens[b], page_size)
        return dequantize_e4m3(kb, k_scale), dequantize_e4m3(vb, v_scale)

    if pairs is None:
        o = np.zeros((B, H, D))
        lse = np.full((B, H), -np.inf)
        for b in range(B):
            kv, vv = rows(b)
            o[b], lse[b] = decode_attention(q[b], kv, vv, scale)
        return o, lse
    pairs = [(int(b), int(h)) for b, h in pairs]
    o = np.zeros((len(pairs), D))
    lse = np.full(len(pairs), -np.inf)
    by_seq: dict[int, list[int]] = {}
    for i, (b, _) in enumerate(pairs):
        by_seq.setdefault(b, []).append(i)
    for b, idx in by_seq.items():  # one gather and dequantisation per sequence
        kv, vv = rows(b)
        oo, ll = decode_attention(q[b], kv, vv, scale, heads=[pairs[i][1] for i in idx])
        o[idx], lse[idx] = oo, ll
    return o, lse
