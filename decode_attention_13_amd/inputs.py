"""Seeded synthetic inputs for single-query decode attention.

This module holds no attention arithmetic: it only draws random numbers, casts
them to the storage dtype, and does the page bookkeeping of a paged KV cache
(page counts, a shuffled page permutation, the padded block table). The float64
oracle (through the tests) and the HIP path both consume what it returns; it
imports neither of them.

Workloads (all seeded, N(0,1) values drawn in float32 and rounded to the storage
dtype with round-to-nearest-even):

* single decode, contiguous KV: ``q[H, D]``, ``k, v[S, Hkv, D]`` -- the problem
  statement of "[CUDA 优化实战] 纯手搓 flash decoding sm120", section
  "1. flash decoding" (q as [head, dim], kv as [seq, head, dim]).
* batched paged decode: ``q[B, H, D]``, ``k_cache, v_cache[num_pages, page_size,
  Hkv, D]``, ``block_table[B, max_blocks]`` (int32, padded with -1),
  ``seq_lens[B]`` -- the layout of "FlashAttention 与推理算子", section
  "一个分页 decode attention kernel（支持 GQA）"; its harness shuffles the
  physical pages and hands them to the sequences in order, which is what
  ``paged_inputs`` does with its own generator.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# Elements drawn per independent child stream; bounds host memory while
# generating multi-GB caches and lets the chunks be drawn in parallel.
CHUNK_ELEMS = 1 << 22

# Child-stream order below each workload seed. Fixed so that a workload's
# tensors do not change when another one is added.
_CHILD = {"q": 0, "k": 1, "v": 2, "lens": 3, "perm": 4, "peak": 5}


def _child(seed_seq: np.random.SeedSequence, *key: int) -> np.random.SeedSequence:
    """Deterministic child of ``seed_seq`` addressed by ``key`` (no spawn state)."""
    return np.random.SeedSequence(entropy=seed_seq.entropy,
                                  spawn_key=tuple(seed_seq.spawn_key) + tuple(key))


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(seed_seq: np.random.SeedSequence, shape, dtype: str) -> torch.Tensor:
    """N(0,1) float32 draws rounded (RNE) to ``dtype``; a contiguous CPU tensor.

    Chunk ``i`` of ``CHUNK_ELEMS`` elements comes from child stream ``i``, so the
    result does not depend on the number of worker threads.
    """
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = torch.empty(n, dtype=DTYPES[dtype])
    nchunks = (n + CHUNK_ELEMS - 1) // CHUNK_ELEMS

    def fill(i: int) -> None:
        lo = i * CHUNK_ELEMS
        hi = min(n, lo + CHUNK_ELEMS)
        rng = np.random.default_rng(_child(seed_seq, i))
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi].copy_(torch.from_numpy(x))  # float32 -> dtype, round to nearest even

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.view(shape)


def default_scale(D: int) -> float:
    """The float32 value of 1/sqrt(D), the pages' default softmax scale."""
    return float(np.float32(1.0 / math.sqrt(D)))


# --------------------------------------------------------------------------- single


def single_inputs(H: int, Hkv: int, S: int, D: int, dtype: str, seed, *,
                  peak_frac: float = 0.0, peak_mult: float = 8.0) -> dict:
    """Contiguous single-decode inputs.

    ``peak_frac`` > 0 picks ``round(peak_frac * S)`` token rows without
    replacement and multiplies every head of those K rows by ``peak_mult`` (a
    power of two, so the product is exact in the storage dtype): a peaked
    softmax. V and q are untouched.
    """
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    q = normal(_child(ss, _CHILD["q"]), (H, D), dtype)
    k = normal(_child(ss, _CHILD["k"]), (S, Hkv, D), dtype)
    v = normal(_child(ss, _CHILD["v"]), (S, Hkv, D), dtype)
    peak_rows = np.zeros(0, dtype=np.int64)
    if peak_frac > 0 and S > 0:
        n_peak = int(round(peak_frac * S))
        rng = np.random.default_rng(_child(ss, _CHILD["peak"]))
        peak_rows = np.sort(rng.choice(S, size=n_peak, replace=False))
        idx = torch.from_numpy(peak_rows)
        k[idx] = k[idx] * peak_mult
    return {"kind": "single", "q": q, "k": k, "v": v, "H": H, "Hkv": Hkv, "S": S,
            "D": D, "dtype": dtype, "scale": default_scale(D), "peak_rows": peak_rows}


# --------------------------------------------------------------------------- paged


def page_table(seq_lens, page_size: int, perm_seed) -> tuple[np.ndarray, int, int]:
    """Shuffled physical pages handed to the sequences in order.

    Returns ``(block_table[B, max_blocks] int32 padded with -1, num_pages,
    max_blocks)``. The pool holds exactly ``sum(ceil(L_b / page_size))`` pages.
    ``perm_seed`` None gives the identity assignment (pages in sequence order).
    """
    lens = [int(x) for x in seq_lens]
    counts = [(L + page_size - 1) // page_size for L in lens]
    num_pages = int(sum(counts))
    max_blocks = max([1] + counts)
    if perm_seed is None:
        perm = np.arange(num_pages, dtype=np.int64)
    else:
        ss = perm_seed if isinstance(perm_seed, np.random.SeedSequence) else np.random.SeedSequence(perm_seed)
        perm = np.random.default_rng(ss).permutation(num_pages)
    table = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    nxt = 0
    for b, c in enumerate(counts):
        table[b, :c] = perm[nxt:nxt + c]
        nxt += c
    return table, num_pages, max_blocks


def lengths(kind: str, B: int, lo: int, hi: int, seed_seq) -> np.ndarray:
    """Sequence lengths: ``uniform`` integers on [lo, hi] inclusive, or
    ``loguniform``: clamp(round(exp(U(ln lo, ln hi))), lo, hi)."""
    rng = np.random.default_rng(seed_seq)
    if kind == "uniform":
        return rng.integers(lo, hi + 1, size=B).astype(np.int32)
    if kind == "loguniform":
        x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=B))
        return np.clip(np.rint(x), lo, hi).astype(np.int32)
    raise ValueError(kind)


def paged_inputs(B: int, H: int, Hkv: int, D: int, dtype: str, page_size: int, seq_lens,
                 seed, *, shuffle: bool = True) -> dict:
    """Paged GQA decode inputs over a pool of exactly the pages the lengths need.

    Every slot of the pool, including the tail slots past ``L_b`` in a sequence's
    last page, holds an N(0,1) draw.
    """
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    lens = np.asarray(seq_lens, dtype=np.int32)
    table, num_pages, max_blocks = page_table(lens, page_size, _child(ss, _CHILD["perm"]) if shuffle else None)
    q = normal(_child(ss, _CHILD["q"]), (B, H, D), dtype)
    pages = max(num_pages, 1)
    k_cache = normal(_child(ss, _CHILD["k"]), (pages, page_size, Hkv, D), dtype)
    v_cache = normal(_child(ss, _CHILD["v"]), (pages, page_size, Hkv, D), dtype)
    return {"kind": "paged", "q": q, "k_cache": k_cache, "v_cache": v_cache,
            "block_table": torch.from_numpy(table), "seq_lens": torch.from_numpy(lens.copy()),
            "B": B, "H": H, "Hkv": Hkv, "D": D, "dtype": dtype, "page_size": page_size,
            "num_pages": pages, "max_blocks": max_blocks, "max_seq_len": int(lens.max()) if len(lens) else 0,
            "total_kv": int(lens.astype(np.int64).sum()), "scale": default_scale(D)}


# --------------------------------------------------------------------------- FP8 KV

FP8_SCALE = 1.0 / 16.0  # per-tensor dequantisation scale of the synthetic FP8 caches


def to_e4m3(x: torch.Tensor, scale: float) -> torch.Tensor:
    """FP8 E4M3 codes of x / scale (round to nearest even, clamped to +-448)."""
    return (x.float() / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)


def with_fp8_kv(d: dict, scale: float = FP8_SCALE) -> dict:
    """The same workload with its K/V (or caches) stored as E4M3 codes, q kept.

    The codes quantise the original N(0,1) draws; ``k_scale``/``v_scale`` map
    them back. NaN poison (used by the paging tests) stays NaN.
    """
    out = dict(d)
    for key in ("k", "v", "k_cache", "v_cache"):
        if key in d:
            out[key] = to_e4m3(d[key], scale)
    out["k_scale"] = scale
    out["v_scale"] = scale
    out["kv_dtype"] = "fp8"
    return out


# --------------------------------------------------------------------------- workloads


@dataclass(frozen=True)
class SingleWorkload:
    name: str
    index: int
    H: int
    Hkv: int
    S: int
    D: int
    dtype: str
    peak_frac: float = 0.0

    kind = "single"

    def make(self) -> dict:
        return single_inputs(self.H, self.Hkv, self.S, self.D, self.dtype,
                             np.random.SeedSequence(1000 + self.index), peak_frac=self.peak_frac)

    def kv_bytes(self) -> int:
        return 2 * self.S * self.Hkv * self.D * torch.tensor([], dtype=DTYPES[self.dtype]).element_size()


@dataclass(frozen=True)
class PagedWorkload:
    name: str
    index: int
    B: int
    H: int
    Hkv: int
    D: int
    dtype: str
    page_size: int
    len_kind: str
    len_lo: int
    len_hi: int

    kind = "paged"

    def seq_lens(self) -> np.ndarray:
        ss = np.random.SeedSequence(1000 + self.index)
        return lengths(self.len_kind, self.B, self.len_lo, self.len_hi, _child(ss, _CHILD["lens"]))

    def make(self) -> dict:
        return paged_inputs(self.B, self.H, self.Hkv, self.D, self.dtype, self.page_size,
                            self.seq_lens(), np.random.SeedSequence(1000 + self.index))

    def kv_bytes(self) -> int:
        esize = torch.tensor([], dtype=DTYPES[self.dtype]).element_size()
        return 2 * int(self.seq_lens().astype(np.int64).sum()) * self.Hkv * self.D * esize


WORKLOADS = {
    w.name: w for w in [
        SingleWorkload("decode_f32_h8_s512", 1, H=8, Hkv=8, S=512, D=128, dtype="f32"),
        SingleWorkload("decode_bf16_h32_s4096", 2, H=32, Hkv=32, S=4096, D=128, dtype="bf16"),
        SingleWorkload("decode_bf16_h32_s131072_peaked", 3, H=32, Hkv=32, S=131072, D=128,
                       dtype="bf16", peak_frac=0.01),
        PagedWorkload("paged_gqa4_bf16_b64_s1k-8k", 4, B=64, H=32, Hkv=8, D=128, dtype="bf16",
                      page_size=16, len_kind="uniform", len_lo=1024, len_hi=8192),
        PagedWorkload("paged_gqa8_f16_b128_s256-64k", 5, B=128, H=64, Hkv=8, D=128, dtype="f16",
                      page_size=16, len_kind="loguniform", len_lo=256, len_hi=65536),
    ]
}

# Group sizes between MHA and the GQA4 batch, for the choice between the vector-ALU
# and the matrix-core split kernels: the GQA4 batch's lengths and page size with 16
# and 24 query heads on its 8 KV heads.
CHOICE_WORKLOADS = {
    w.name: w for w in [
        PagedWorkload("paged_gqa2_bf16_b64_s1k-8k", 4, B=64, H=16, Hkv=8, D=128, dtype="bf16",
                      page_size=16, len_kind="uniform", len_lo=1024, len_hi=8192),
        PagedWorkload("paged_gqa3_bf16_b64_s1k-8k", 4, B=64, H=24, Hkv=8, D=128, dtype="bf16",
                      page_size=16, len_kind="uniform", len_lo=1024, len_hi=8192),
    ]
}


# --------------------------------------------------------------------------- prefill


def prefill_inputs(B: int, N: int, H: int, Hkv: int, D: int, dtype: str, seed) -> dict:
    """q [B, N, H, D], k/v [B, N, Hkv, D] ~ N(0,1) rounded to dtype; scale 1/sqrt(D)."""
    ss = seed if isinstance(seed, np.random.SeedSequence) else np.random.SeedSequence(seed)
    return {"q": normal(_child(ss, 0), (B, N, H, D), dtype), "k": normal(_child(ss, 1), (B, N, Hkv, D), dtype),
            "v": normal(_child(ss, 2), (B, N, Hkv, D), dtype), "scale": default_scale(D)}


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    index: int
    B: int
    N: int
    H: int
    Hkv: int
    D: int
    dtype: str
    causal: bool

    kind = "prefill"

    def make(self) -> dict:
        return prefill_inputs(self.B, self.N, self.H, self.Hkv, self.D, self.dtype,
                              np.random.SeedSequence(1000 + self.index))

    def flops(self) -> int:
        """Useful flops: 4 * D per (query, visible key) pair and head."""
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4 * self.D * pairs * self.B * self.H


# The prompt pass of the same model shapes: 32 heads of 128, a 4k prompt, causal;
# and the GQA-4 shape over two 2k prompts.
PREFILL_WORKLOADS = {
    w.name: w for w in [
        PrefillWorkload("prefill_bf16_h32_n4096_causal", 6, B=1, N=4096, H=32, Hkv=32, D=128, dtype="bf16",
                        causal=True),
        PrefillWorkload("prefill_f16_b2_h32_kv8_n2048_causal", 7, B=2, N=2048, H=32, Hkv=8, D=128, dtype="f16",
                        causal=True),
    ]
}


def sweep_workload(S: int) -> SingleWorkload:
    """The pages' benchmark shape (32 heads, head_dim 128, bf16) at KV length S."""
    return SingleWorkload(f"decode_bf16_h32_s{S}", 100 + S % 1000003, H=32, Hkv=32, S=S, D=128, dtype="bf16")
