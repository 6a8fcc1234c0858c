"""Float64 CPU oracle for single-query decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library and does not import it.

Contents
--------
``decode``  -- the plain definition in numpy float64 (materialises the full
               softmax), the paged gather, split partials and the two merge
               formulas.
``loops``   -- pure-Python three-pass and online-softmax recurrences for tiny
               inputs, used to pin ``decode`` against the pages' step-by-step
               algorithms.
``fp8``     -- values of an FP8 E4M3 KV cache with per-tensor scales, and the
               plain definition over them (contiguous and paged).
``prefill`` -- many-query attention over a prompt with an optional causal mask.

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (the pages' worked example, closed forms, a library routine,
brute force); no function here is "parity unpinned".
"""
from .decode import (  # noqa: F401
    kv_head_of,
    scores,
    softmax_weights,
    log_sum_exp,
    weighted_sum,
    decode_attention,
    gather_pages,
    paged_decode_attention,
    split_bounds,
    split_partials,
    paged_split_partials,
    merge_lse,
    merge_m_l,
)
from . import loops  # noqa: F401
from .prefill import causal_mask, prefill_attention  # noqa: F401
from .fp8 import (  # noqa: F401
    dequantize_e4m3,
    e4m3_value,
    decode_attention_e4m3,
    paged_decode_attention_e4m3,
)
