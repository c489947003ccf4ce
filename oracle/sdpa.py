"""Plain float64 CPU oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes (all arithmetic in float64 on exactly upcast inputs):

* ``attend`` / ``attention`` -- the plain definition O = softmax(S) V with
  S = scale * Q K^T and a row-max-subtracted softmax over the allowed keys
  ("Attention 在算什么", section 1, and the max-subtracting ``softmax_safe``
  of section 4 of the 10100.com article).  A row with no allowed key is 0.
* ``gather_paged`` / ``paged_decode`` -- the block-table walk of the paged
  variant (llminference.xinbetween.com S12, "实现"), with grouped-query head
  sharing (S12, "它如何与你已经搭好的部分组合").
* ``online_partial`` / ``online_attention`` / ``online_attention_q_outer`` --
  the online-softmax recurrence (10100.com section 7; S12 "核心思路"; the
  5688vip example's outer-Q / inner-KV order), started from a finite sentinel
  as S12 recommends against exp(-inf - -inf).
* ``merge_partials`` / ``split_key_attention`` -- combining (m, l, o) states
  of disjoint key ranges (S12 flash-decoding and exercise 1).
* ``paged_prefill`` -- a chunk of query tokens at the end of each sequence
  over the same paged cache (bottom-right aligned causal mask).
* ``attention_range`` / ``merge_lse`` -- the definition restricted to a key
  range, reported as the range's normalised output and the natural log of its
  softmax denominator (log-sum-exp), and the merge of such pieces.  This is
  the (m, l, o) state of S12's split over key ranges ("除了快，它还解锁了
  什么": ring attention and flash-decoding exchange exactly these partial
  states) written as (o, lse) with lse = m + log l.

Readings of points the pages leave open:
* scale is explicit; callers pass 1/sqrt(d) (10100.com section 2, S12) or 1
  (the 5688vip example omits it);
* causal means key j is allowed for query i iff j <= i (top-left aligned);
* a left-padded sequence b of length L_b occupies positions [N - L_b, N) of
  both queries and keys; rows before that are padding and produce zeros;
* masked and padded entries never enter the arithmetic (they are sliced or
  selected away), so poison values there cannot leak.
"""
from __future__ import annotations

import numpy as np

# A large finite negative start for the running max (S12: initialise the max
# with a big finite negative number so a fully masked first tile gives
# exp(-inf - sentinel) = 0 instead of exp(nan)).
SENTINEL = -1.0e300


# --------------------------------------------------------------------------
# The definition
# --------------------------------------------------------------------------
def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q [r, d], k [m, d] -> [r, m]."""
    return (q @ k.T) * scale


def allowed_keys(row_idx: np.ndarray, key_idx: np.ndarray, causal: bool, pad: int) -> np.ndarray:
    """Boolean [r, m]: may query row_idx[a] attend key key_idx[b]?"""
    ok = np.ones((row_idx.size, key_idx.size), dtype=bool)
    if causal:
        ok &= key_idx[None, :] <= row_idx[:, None]
    ok &= key_idx[None, :] >= pad
    ok &= row_idx[:, None] >= pad
    return ok


def masked_softmax(s: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """Row softmax over the allowed entries, subtracting the row max first
    (10100.com section 4).  Rows with no allowed entry are all zero."""
    s = np.where(ok, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    has = np.isfinite(mx)
    mx = np.where(has, mx, 0.0)
    e = np.where(ok, np.exp(s - mx), 0.0)
    den = e.sum(axis=1, keepdims=True)
    return np.where(has, e / np.where(has, den, 1.0), 0.0)


def attend(q_rows: np.ndarray, row_idx, k: np.ndarray, v: np.ndarray, scale: float,
           causal: bool = False, pad: int = 0) -> np.ndarray:
    """Output rows of one head.

    q_rows [r, d] are the queries at absolute positions ``row_idx``; k [m, d],
    v [m, dv] are the head's keys and values; keys before ``pad`` are padding
    and are never read.
    """
    row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
    m = k.shape[0]
    key_idx = np.arange(pad, m, dtype=np.int64)
    ks, vs = k[pad:], v[pad:]
    s = scores(q_rows, ks, scale)
    p = masked_softmax(s, allowed_keys(row_idx, key_idx, causal, pad))
    return p @ vs


def probabilities(q: np.ndarray, k: np.ndarray, scale: float, causal: bool = False,
                  pad: int = 0) -> np.ndarray:
    """P [n, m - pad] of one head (the 5688vip ``standard_attention`` also
    returns P); used for the row-sum invariant."""
    n = q.shape[0]
    row_idx = np.arange(n)
    key_idx = np.arange(pad, k.shape[0])
    return masked_softmax(scores(q, k[pad:], scale), allowed_keys(row_idx, key_idx, causal, pad))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal: bool = False,
              pads=None, chunk: int = 1024) -> np.ndarray:
    """Batched definition: q [B, Hq, n, d], k [B, Hkv, m, d], v [B, Hkv, m, dv]
    -> O [B, Hq, n, dv].  Query head h reads KV head h // (Hq // Hkv).
    ``pads``: None or per-batch count of leading padding positions."""
    B, Hq, n, _ = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, n, v.shape[3]), dtype=np.float64)
    for b in range(B):
        pad = 0 if pads is None else int(pads[b])
        for h in range(Hq):
            kh, vh = k[b, h // group], v[b, h // group]
            for r0 in range(pad, n, chunk):
                r1 = min(n, r0 + chunk)
                out[b, h, r0:r1] = attend(q[b, h, r0:r1], np.arange(r0, r1), kh, vh,
                                          scale, causal, pad)
    return out


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, samples,
                   causal: bool = False, pads=None) -> np.ndarray:
    """O at sampled positions: ``samples`` is a list of (b, h, i); returns [S, dv]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    group = Hq // Hkv
    out = np.zeros((len(samples), v.shape[-1]), dtype=np.float64)
    for t, (b, h, i) in enumerate(samples):
        pad = 0 if pads is None else int(pads[b])
        if i < pad:
            continue
        out[t] = attend(q[b, h, i][None, :], [i], k[b, h // group], v[b, h // group],
                        scale, causal, pad)[0]
    return out


# --------------------------------------------------------------------------
# Paged decode
# --------------------------------------------------------------------------
def gather_paged(cache: np.ndarray, table_row, seq_len: int, block_size: int, head: int) -> np.ndarray:
    """Rows of one KV head in logical order: walk the block table, take
    min(block_size, seq_len - t * block_size) slots of block t, stop at the
    first block with none (S12 "实现").  cache [NB, bs, Hkv, d]."""
    rows = []
    for logical, physical in enumerate(table_row):
        cnt = min(block_size, int(seq_len) - logical * block_size)
        if cnt <= 0:
            break
        rows.append(cache[int(physical), :cnt, head])
    if not rows:
        return np.zeros((0, cache.shape[-1]), dtype=cache.dtype)
    return np.concatenate(rows, axis=0)


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table,
                 seq_lens, block_size: int, scale: float) -> np.ndarray:
    """One query token per sequence over a paged, grouped-query KV cache.
    q [S, Hq, d] -> O [S, Hq, dv]; query head h reads KV head h // (Hq // Hkv)."""
    S, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    out = np.zeros((S, Hq, v_cache.shape[-1]), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        for g in range(Hkv):
            kg = gather_paged(k_cache, block_table[s], L, block_size, g)
            vg = gather_paged(v_cache, block_table[s], L, block_size, g)
            heads = slice(g * group, (g + 1) * group)
            out[s, heads] = attend(q[s, heads], np.full(group, L - 1), kg, vg, scale)
    return out


def paged_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table,
                  seq_lens, block_size: int, scale: float, causal: bool = True) -> np.ndarray:
    """A chunk of n query tokens per sequence over a paged, grouped-query KV
    cache that already holds the chunk's own keys: q [S, Hq, n, d] ->
    O [S, Hq, n, dv].  Query row i of sequence s is token L_s - n + i, so the
    chunk is the last n tokens of the sequence; with ``causal`` it attends
    keys 0 .. L_s - n + i, else all L_s keys.  Rows at negative positions
    (n > L_s) have no keys and give 0.  The keys are the block-table walk of
    S12 "实现" (the chapter notes each tile can come through the block table);
    n = 1 is ``paged_decode``."""
    S, Hq, n, _ = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    out = np.zeros((S, Hq, n, v_cache.shape[-1]), dtype=np.float64)
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        pos = np.arange(L - n, L, dtype=np.int64)
        live = pos >= 0
        for g in range(Hkv):
            kg = gather_paged(k_cache, block_table[s], L, block_size, g)
            vg = gather_paged(v_cache, block_table[s], L, block_size, g)
            for h in range(g * group, (g + 1) * group):
                if causal:
                    out[s, h, live] = attend(q[s, h, live], pos[live], kg, vg, scale, True)
                else:
                    out[s, h, live] = attend(q[s, h, live], pos[live], kg, vg, scale, False)
    return out


# --------------------------------------------------------------------------
# The online-softmax recurrence (a second, independent route to the same
# numbers; the tests hold it against the definition)
# --------------------------------------------------------------------------
def online_partial(q_rows: np.ndarray, row_idx, k: np.ndarray, v: np.ndarray, scale: float,
                   tile: int, key_lo: int = 0, key_hi: int | None = None,
                   causal: bool = False, pad: int = 0):
    """Run the recurrence over keys [key_lo, key_hi) in tiles of ``tile`` keys.

    State per row: m (running max, from the finite sentinel), l (sum of
    exponentials rescaled to m) and acc (weighted sum of values rescaled to
    m).  Each tile: m_new = max(m, tile row max); alpha = exp(m - m_new);
    p = exp(s - m_new); l = alpha*l + sum(p); acc = alpha*acc + p V.
    Returns (m, l, acc).
    """
    row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
    r = q_rows.shape[0]
    key_hi = k.shape[0] if key_hi is None else key_hi
    m_run = np.full(r, SENTINEL)
    l_run = np.zeros(r)
    acc = np.zeros((r, v.shape[1]))
    for j0 in range(key_lo, key_hi, tile):
        j1 = min(key_hi, j0 + tile)
        key_idx = np.arange(j0, j1)
        lo = max(j0, pad)
        s = np.full((r, j1 - j0), -np.inf)
        if lo < j1:
            s[:, lo - j0:] = scores(q_rows, k[lo:j1], scale)
        ok = allowed_keys(row_idx, key_idx, causal, pad)
        s = np.where(ok, s, -np.inf)
        m_new = np.maximum(m_run, s.max(axis=1))
        alpha = np.exp(m_run - m_new)
        p = np.exp(s - m_new[:, None])
        l_run = alpha * l_run + p.sum(axis=1)
        vt = np.zeros((j1 - j0, v.shape[1]))
        if lo < j1:
            vt[lo - j0:] = v[lo:j1]
        acc = alpha[:, None] * acc + p @ vt
        m_run = m_new
    return m_run, l_run, acc


def finish(m_run, l_run, acc) -> np.ndarray:
    """O = acc / l, with rows that saw no allowed key set to 0."""
    safe = np.where(l_run > 0, l_run, 1.0)
    return np.where((l_run > 0)[:, None], acc / safe[:, None], 0.0)


def online_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, tile: int,
                     causal: bool = False, pad: int = 0) -> np.ndarray:
    """One head, all query rows as one block, keys in tiles (10100.com v4 order)."""
    n = q.shape[0]
    return finish(*online_partial(q, np.arange(n), k, v, scale, tile, causal=causal, pad=pad))


def online_attention_q_outer(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                             q_block: int, k_block: int, causal: bool = False,
                             pad: int = 0) -> np.ndarray:
    """One head, query blocks outside and key blocks inside (the 5688vip order);
    every query block keeps its own (m, l, acc) and is normalised at the end."""
    n = q.shape[0]
    out = np.zeros((n, v.shape[1]))
    for i0 in range(0, n, q_block):
        i1 = min(n, i0 + q_block)
        out[i0:i1] = finish(*online_partial(q[i0:i1], np.arange(i0, i1), k, v, scale, k_block,
                                            causal=causal, pad=pad))
    return out


def merge_partials(parts) -> np.ndarray:
    """Combine (m, l, acc) states of disjoint key ranges: with M = max m_s and
    w_s = exp(m_s - M), O = sum w_s acc_s / sum w_s l_s (the same rescale the
    recurrence applies; S12 exercise 1)."""
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    l_tot = np.zeros_like(parts[0][1])
    acc_tot = np.zeros_like(parts[0][2])
    for m_s, l_s, acc_s in parts:
        w = np.exp(m_s - M)
        l_tot = l_tot + w * l_s
        acc_tot = acc_tot + w[:, None] * acc_s
    return finish(M, l_tot, acc_tot)


def split_key_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, bounds,
                        tile: int, causal: bool = False, pad: int = 0) -> np.ndarray:
    """Flash-decoding on the CPU: run the recurrence independently on each key
    range [bounds[t], bounds[t+1]) and merge the states."""
    n = q.shape[0]
    parts = [online_partial(q, np.arange(n), k, v, scale, tile, lo, hi, causal, pad)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    return merge_partials(parts)


# --------------------------------------------------------------------------
# Key-range pieces and their merge (S12 split over key ranges, exercise 1)
# --------------------------------------------------------------------------
def attention_range(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                    causal: bool = False, pads=None, key_begin: int = 0, key_end=None):
    """The definition over the allowed keys that also lie in [key_begin, key_end).

    Returns (O [B, Hq, n, dv], lse [B, Hq, n]): O is the softmax-weighted mean
    of those keys' values and lse = log(sum exp(s_ij)) over them, computed as
    max + log(sum exp(s - max)).  A row with no such key has O = 0 and
    lse = -inf.  Keys outside the range are never read.
    """
    B, Hq, n, _ = q.shape
    Hkv, m = k.shape[1], k.shape[2]
    group = Hq // Hkv
    key_end = m if key_end is None else min(int(key_end), m)
    out = np.zeros((B, Hq, n, v.shape[3]))
    lse = np.full((B, Hq, n), -np.inf)
    for b in range(B):
        pad = 0 if pads is None else int(pads[b])
        lo = max(int(key_begin), pad)
        if lo >= key_end:
            continue
        key_idx = np.arange(lo, key_end, dtype=np.int64)
        row_idx = np.arange(n, dtype=np.int64)
        for h in range(Hq):
            ks, vs = k[b, h // group, lo:key_end], v[b, h // group, lo:key_end]
            s = scores(q[b, h], ks, scale)
            ok = allowed_keys(row_idx, key_idx, causal, pad)
            s = np.where(ok, s, -np.inf)
            mx = s.max(axis=1)
            has = np.isfinite(mx)
            mx0 = np.where(has, mx, 0.0)
            e = np.where(ok, np.exp(s - mx0[:, None]), 0.0)
            den = e.sum(axis=1)
            out[b, h] = np.where(has[:, None], (e @ vs) / np.where(has, den, 1.0)[:, None], 0.0)
            lse[b, h] = np.where(has, mx0 + np.log(np.where(has, den, 1.0)), -np.inf)
    return out, lse


def merge_lse(parts):
    """Merge (O_s, lse_s) pieces of disjoint key ranges into (O, lse).

    With L = max_s lse_s and w_s = exp(lse_s - L): O = sum w_s O_s / sum w_s
    and lse = L + log(sum w_s) -- the rescale of the recurrence applied to
    whole pieces (S12 exercise 1), since O_s = acc_s / l_s and lse_s = m_s +
    log l_s.  Pieces with lse_s = -inf weigh 0; if all are -inf, O = 0.
    """
    lses = np.stack([p_[1] for p_ in parts])
    L = lses.max(axis=0)
    has = np.isfinite(L)
    L0 = np.where(has, L, 0.0)
    w_tot = np.zeros_like(L0)
    o_tot = np.zeros_like(parts[0][0], dtype=np.float64)
    for o_s, lse_s in parts:
        w = np.where(np.isfinite(lse_s), np.exp(np.where(np.isfinite(lse_s), lse_s, 0.0) - L0), 0.0)
        w_tot = w_tot + w
        o_tot = o_tot + w[..., None] * o_s
    o = np.where(has[..., None], o_tot / np.where(has, w_tot, 1.0)[..., None], 0.0)
    lse = np.where(has, L0 + np.log(np.where(has, w_tot, 1.0)), -np.inf)
    return o, lse
