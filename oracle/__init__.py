"""CPU float64 oracle for tiled online-softmax attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``, never by the HIP library or its
Python binding.  See ``oracle/sdpa.py`` for what each function follows.
"""
from .sdpa import (SENTINEL, allowed_keys, attend, attention, attention_range, attention_rows,
                   finish, gather_paged, masked_softmax, merge_lse, merge_partials,
                   online_attention, online_attention_q_outer, online_partial, paged_decode,
                   paged_prefill, probabilities, scores, split_key_attention)

__all__ = [
    "SENTINEL", "allowed_keys", "attend", "attention", "attention_range", "attention_rows",
    "finish", "gather_paged", "masked_softmax", "merge_lse", "merge_partials",
    "online_attention",
    "online_attention_q_outer", "online_partial", "paged_decode", "paged_prefill",
    "probabilities", "scores",
    "split_key_attention",
]
