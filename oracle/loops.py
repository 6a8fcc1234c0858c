"""Pure-Python recurrences for tiny inputs (lists of floats, Python double).

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``three_pass``: the three steps of the paged decode kernel in "FlashAttention
  与推理算子", section "一个分页 decode attention kernel（支持 GQA）": all
  scores and their max, then the exponentials and their sum, then the
  probability-weighted sum of the values.
* ``online``: the blockwise recurrence of the same page, section
  "FlashAttention：分块 + online softmax": per block j, m_j = max(m_{j-1},
  rowmax S_j), P~_j = exp(S_j - m_j), l_j = e^{m_{j-1} - m_j} l_{j-1} +
  rowsum P~_j, O_j = e^{m_{j-1} - m_j} O_{j-1} + P~_j V_j; the result is
  O_last / l_last.

These are only used on inputs small enough to check by hand (a handful of keys
and dimensions).
"""
from __future__ import annotations

import math


def _dot(a, b) -> float:
    return sum(float(x) * float(y) for x, y in zip(a, b))


def three_pass(q, keys, values, scale: float):
    """Returns ``(o, lse)``: o a list of len(values[0]) floats."""
    n = len(keys)
    if n == 0:
        return [0.0] * (len(values[0]) if values else 0), -math.inf
    s = [_dot(q, kt) * scale for kt in keys]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    total = sum(e)
    dim = len(values[0])
    o = [sum(e[t] * float(values[t][d]) for t in range(n)) / total for d in range(dim)]
    return o, mx + math.log(total)


def online(q, keys, values, scale: float, block: int, trace: list | None = None):
    """Blockwise online softmax. ``trace`` (if given) receives (m, l, O) after each block.

    Returns ``(o, lse)``.
    """
    dim = len(values[0]) if values else 0
    m = -math.inf
    l = 0.0
    O = [0.0] * dim
    for j0 in range(0, len(keys), block):
        kb = keys[j0:j0 + block]
        vb = values[j0:j0 + block]
        s = [_dot(q, kt) * scale for kt in kb]
        m_new = max(m, max(s))
        corr = math.exp(m - m_new)  # 0 on the first block (m = -inf)
        p = [math.exp(x - m_new) for x in s]
        l = corr * l + sum(p)
        O = [corr * O[d] + sum(p[t] * float(vb[t][d]) for t in range(len(kb))) for d in range(dim)]
        m = m_new
        if trace is not None:
            trace.append((m, l, list(O)))
    if l == 0.0:
        return [0.0] * dim, -math.inf
    return [x / l for x in O], m + math.log(l)


def online_from_scores(score_blocks, value_blocks, trace: list | None = None):
    """The same recurrence fed with precomputed score blocks and scalar values.

    This is the form of the hand-worked exercise (scores [1, 3] then [2, 5],
    values [10, 20] then [30, 40]). Returns the final O / l.
    """
    m = -math.inf
    l = 0.0
    O = 0.0
    for s, vals in zip(score_blocks, value_blocks):
        m_new = max(m, max(s))
        corr = math.exp(m - m_new)
        p = [math.exp(x - m_new) for x in s]
        l = corr * l + sum(p)
        O = corr * O + sum(pi * vi for pi, vi in zip(p, vals))
        if trace is not None:
            trace.append({"m": m_new, "correction": corr, "p": list(p), "l": l, "O": O})
        m = m_new
    return O / l
