"""CPU float64 oracle for tiled online-softmax attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``, never by the HIP library or its
Python binding.  See ``oracle/sdpa.py`` for what each function follows, and
``oracle/fp8.py`` for the FP8 (E4M3) inputs.
"""
from .sdpa import (SENTINEL, allowed_keys, attend, attention, attention_range, attention_rows,
                   finish, gather_paged, masked_softmax, merge_lse, merge_partials,
                   online_attention, online_attention_q_outer, online_partial, paged_decode,
                   paged_prefill, probabilities, scores, split_key_attention)
from .fp8 import attention_fp8, dequantize, e4m3_to_f64

__all__ = [
    "attention_fp8", "dequantize", "e4m3_to_f64",
    "SENTINEL", "allowed_keys", "attend", "attention", "attention_range", "attention_rows",
    "finish", "gather_paged", "masked_softmax", "merge_lse", "merge_partials",
    "online_attention",
    "online_attention_q_outer", "online_partial", "paged_decode", "paged_prefill",
    "probabilities", "scores",
    "split_key_attention",
]
