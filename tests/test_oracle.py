"""Pins for the float64 oracle (CPU only).

Each check ties the oracle to something other than itself: brute force on tiny
inputs, the recurrence of the pages at many tile sizes, the 5688vip self-test,
closed forms, invariants, a library softmax, and negative controls that must
fail.  ``test_pins_catch_planted_mistakes`` plants plausible mistakes in the
oracle and requires at least one pin to catch each.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.sdpa as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLDEN, "page_figures.json")) as f:
    FIG = json.load(f)

TIGHT = 1e-12


def rnd(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# --------------------------------------------------------------------------
# brute force: the definition as literal loops (10100.com version 0 shape:
# per query, per key dot product times the scale, softmax, weighted sum into a
# float64 accumulator), with the mask written out per (i, j)
# --------------------------------------------------------------------------
def brute_force(q, k, v, scale, causal=False, pad=0):
    n, d = q.shape
    m, dv = v.shape
    out = np.zeros((n, dv))
    for i in range(n):
        allowed = [j for j in range(m)
                   if (not causal or j <= i) and j >= pad and i >= pad]
        if not allowed:
            continue
        sc = {}
        for j in allowed:
            acc = 0.0
            for t in range(d):
                acc += float(q[i, t]) * float(k[j, t])
            sc[j] = acc * scale
        w = {j: math.exp(sc[j]) for j in allowed}  # naive exp: fine on N(0,1) data
        tot = sum(w.values())
        for j in allowed:
            for c in range(dv):
                out[i, c] += w[j] / tot * float(v[j, c])
    return out


def brute_force_paged(q, k_cache, v_cache, table, seq_lens, bs, scale):
    S, Hq, _ = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((S, Hq, v_cache.shape[-1]))
    for s in range(S):
        L = int(seq_lens[s])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            if L == 0:
                continue
            ks = np.array([k_cache[table[s, t // bs], t % bs, g] for t in range(L)])
            vs = np.array([v_cache[table[s, t // bs], t % bs, g] for t in range(L)])
            out[s, h] = brute_force(q[s, h][None], ks, vs, scale)[0]
    return out


def make_paged(rng, S=3, Hq=4, Hkv=2, d=5, dv=6, bs=4, lens=(0, 7, 12), maxb=4):
    nblk = [(L + bs - 1) // bs for L in lens]
    NB = sum(nblk) + 2
    kc = rnd(rng, NB, bs, Hkv, d)
    vc = rnd(rng, NB, bs, Hkv, dv)
    perm = rng.permutation(NB)
    table = np.full((S, maxb), -1, dtype=np.int64)
    pos = 0
    for s in range(S):
        table[s, :nblk[s]] = perm[pos:pos + nblk[s]]
        pos += nblk[s]
    q = rnd(rng, S, Hq, d)
    return q, kc, vc, table, np.array(lens), bs


# --------------------------------------------------------------------------
# pin bodies, reusable by the planted-mistake test (each returns True on pass)
# --------------------------------------------------------------------------
def pin_bruteforce_prefill():
    rng = np.random.default_rng(11)
    ok = True
    for (n, m, d, dv, causal, pad) in [(5, 7, 3, 4, False, 0), (6, 6, 4, 2, True, 0),
                                      (7, 7, 3, 3, True, 3), (6, 6, 2, 5, False, 2),
                                      (1, 1, 8, 8, True, 0), (4, 9, 8, 3, False, 0)]:
        q, k, v = rnd(rng, n, d), rnd(rng, m, d), rnd(rng, m, dv)
        scale = 1.0 / math.sqrt(d)
        got = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal,
                               pads=None if pad == 0 else [pad])[0, 0]
        ok &= np.abs(got - brute_force(q, k, v, scale, causal, pad)).max() <= TIGHT
    return bool(ok)


def pin_bruteforce_gqa():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, n, d, dv = 2, 4, 2, 5, 3, 4
    q, k, v = rnd(rng, B, Hq, n, d), rnd(rng, B, Hkv, n, d), rnd(rng, B, Hkv, n, dv)
    got = oracle.attention(q, k, v, 0.7, causal=True, pads=[0, 2])
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            ref = brute_force(q[b, h], k[b, h // 2], v[b, h // 2], 0.7, True, [0, 2][b])
            worst = max(worst, np.abs(got[b, h] - ref).max())
    return worst <= TIGHT


def pin_bruteforce_paged():
    rng = np.random.default_rng(13)
    q, kc, vc, table, lens, bs = make_paged(rng)
    got = oracle.paged_decode(q, kc, vc, table, lens, bs, 0.5)
    return np.abs(got - brute_force_paged(q, kc, vc, table, lens, bs, 0.5)).max() <= TIGHT


def pin_causal_row0():
    rng = np.random.default_rng(14)
    q, k, v = rnd(rng, 9, 4), rnd(rng, 9, 4), rnd(rng, 9, 3)
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, causal=True)[0, 0]
    return bool(np.array_equal(o[0], v[0]))


def pin_causal_prefix_means():
    rng = np.random.default_rng(15)
    n = 11
    v = rnd(rng, n, 3)
    q = np.zeros((n, 4))
    k = rnd(rng, n, 4)
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3, causal=True)[0, 0]
    expect = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    return np.abs(o - expect).max() <= TIGHT


def pin_hot_finite():
    # scores far past float64's exp overflow (about 709): the result must
    # stay finite and within the range of V
    rng = np.random.default_rng(16)
    q, k, v = rnd(rng, 32, 64, scale=40.0), rnd(rng, 32, 64, scale=40.0), rnd(rng, 32, 64)
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 1 / 8, causal=False)[0, 0]
    assert np.abs(oracle.scores(q, k, 1 / 8)).max() > 709
    return bool(np.isfinite(o).all() and np.all(o <= v.max(0) + 1e-12)
                and np.all(o >= v.min(0) - 1e-12))


def pin_dominant_key():
    # one key's score exceeds every other by >= 50: O is that key's V row
    # (within exp(-50)); the scores also exceed float64's exp range
    rng = np.random.default_rng(34)
    k = rnd(rng, 12, 16)
    v = rnd(rng, 12, 6)
    j = 7
    q = (k[j] * 60.0)[None, :]
    s = oracle.scores(q, k, 1.0)[0]
    if s[j] - np.delete(s, j).max() < 50 or s[j] < 709:
        return False
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 1.0)[0, 0, 0]
    return bool(np.abs(o - v[j]).max() < TIGHT)


def pin_recurrence_sweep():
    rng = np.random.default_rng(17)
    ok = True
    for causal, pad in [(False, 0), (True, 0), (True, 5), (False, 5)]:
        n, d, dv = 37, 6, 5
        q, k, v = rnd(rng, n, d, scale=3.0), rnd(rng, n, d, scale=3.0), rnd(rng, n, dv)
        ref = oracle.attention(q[None, None], k[None, None], v[None, None], 0.4, causal,
                               pads=None if pad == 0 else [pad])[0, 0]
        for tile in (1, 2, 3, 7, 16, 64, n):
            o1 = oracle.online_attention(q, k, v, 0.4, tile, causal, pad)
            o2 = oracle.online_attention_q_outer(q, k, v, 0.4, max(1, tile // 2 + 1), tile,
                                                 causal, pad)
            ok &= np.abs(o1 - ref).max() <= TIGHT and np.abs(o2 - ref).max() <= TIGHT
    return bool(ok)


def pin_split_merge():
    rng = np.random.default_rng(18)
    ok = True
    for trial in range(5):
        n, m, d, dv = 3, 40, 8, 8
        q, k, v = rnd(rng, n, d, scale=2.0), rnd(rng, m, d, scale=2.0), rnd(rng, m, dv)
        cuts = np.sort(rng.integers(0, m + 1, size=3))
        bounds = [0, *cuts.tolist(), m]          # 4 ranges, some may be empty
        ref = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3)[0, 0]
        got = oracle.split_key_attention(q, k, v, 0.3, bounds, tile=5)
        ok &= np.abs(got - ref).max() <= TIGHT
    return bool(ok)


def pin_gqa_equals_repeated_mha():
    rng = np.random.default_rng(19)
    B, Hq, Hkv, n, d = 1, 8, 2, 6, 4
    q, k, v = rnd(rng, B, Hq, n, d), rnd(rng, B, Hkv, n, d), rnd(rng, B, Hkv, n, d)
    g = oracle.attention(q, k, v, 0.5)
    m = oracle.attention(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), 0.5)
    return np.abs(g - m).max() <= TIGHT


def pin_paged_equals_contiguous():
    rng = np.random.default_rng(20)
    S, Hq, Hkv, d, bs = 2, 4, 2, 8, 4
    lens = [9, 16]
    q, kc, vc, table, lens, bs = make_paged(rng, S=2, Hq=Hq, Hkv=Hkv, d=d, dv=d, bs=bs,
                                            lens=lens, maxb=5)
    got = oracle.paged_decode(q, kc, vc, table, lens, bs, 0.35)
    worst = 0.0
    for s in range(S):
        L = int(lens[s])
        # contiguous K/V of the sequence, built by logical token index
        kk = np.stack([kc[table[s, t // bs], t % bs] for t in range(L)], axis=1)  # [Hkv, L, d]
        vv = np.stack([vc[table[s, t // bs], t % bs] for t in range(L)], axis=1)
        ref = oracle.attention(q[s][None, :, None, :], kk[None], vv[None], 0.35)[0, :, 0]
        worst = max(worst, np.abs(got[s] - ref).max())
    return worst <= TIGHT


# --------------------------------------------------------------------------
# key-range pieces (o, lse) and their merge
# --------------------------------------------------------------------------
def brute_force_range(q, k, v, scale, lo, hi, causal=False, pad=0):
    """Literal loops: the allowed keys of row i inside [lo, hi), their
    weighted mean of values and log(sum exp(score))."""
    n, d = q.shape
    dv = v.shape[1]
    out, lse = np.zeros((n, dv)), np.full(n, -np.inf)
    for i in range(n):
        allowed = [j for j in range(max(lo, pad), hi)
                   if (not causal or j <= i) and i >= pad]
        if not allowed:
            continue
        sc = {j: sum(float(q[i, t]) * float(k[j, t]) for t in range(d)) * scale for j in allowed}
        w = {j: math.exp(sc[j]) for j in allowed}
        tot = sum(w.values())
        lse[i] = math.log(tot)
        for j in allowed:
            for c in range(dv):
                out[i, c] += w[j] / tot * float(v[j, c])
    return out, lse


def pin_range_bruteforce():
    rng = np.random.default_rng(21)
    worst = 0.0
    for causal, pad, lo, hi in [(False, 0, 0, 9), (False, 0, 3, 7), (True, 0, 2, 9),
                                (True, 3, 0, 5), (False, 2, 6, 6), (True, 0, 8, 9)]:
        n = m = 9
        q, k, v = rnd(rng, n, 4), rnd(rng, m, 4), rnd(rng, m, 3)
        got_o, got_l = oracle.attention_range(q[None, None], k[None, None], v[None, None], 0.6,
                                              causal, None if pad == 0 else [pad], lo, hi)
        ref_o, ref_l = brute_force_range(q, k, v, 0.6, lo, hi, causal, pad)
        if not np.array_equal(np.isinf(got_l[0, 0]), np.isinf(ref_l)):
            return False
        fin = np.isfinite(ref_l)
        worst = max(worst, np.abs(got_o[0, 0] - ref_o).max(),
                    np.abs(got_l[0, 0][fin] - ref_l[fin]).max(initial=0.0))
    return worst <= TIGHT


def pin_range_merge():
    rng = np.random.default_rng(22)
    worst = 0.0
    for causal, pads in [(False, None), (True, None), (True, [0, 5])]:
        B, Hq, Hkv, n, d = 2, 4, 2, 20, 6
        q = rnd(rng, B, Hq, n, d, scale=2.0)
        k, v = rnd(rng, B, Hkv, n, d, scale=2.0), rnd(rng, B, Hkv, n, d)
        cuts = np.sort(rng.integers(0, n + 1, size=3))
        bounds = [0, *cuts.tolist(), n]
        parts = [oracle.attention_range(q, k, v, 0.4, causal, pads, lo, hi)
                 for lo, hi in zip(bounds[:-1], bounds[1:])]
        o, lse = oracle.merge_lse(parts)
        ref = oracle.attention(q, k, v, 0.4, causal, pads)
        _, lse_full = oracle.attention_range(q, k, v, 0.4, causal, pads)
        if not np.array_equal(np.isinf(lse), np.isinf(lse_full)):
            return False
        fin = np.isfinite(lse_full)
        worst = max(worst, np.abs(o - ref).max(), np.abs(lse[fin] - lse_full[fin]).max())
    return worst <= TIGHT


def pin_range_matches_recurrence():
    """The (o, lse) of a range equals the recurrence's state over the same
    range: o = acc / l and lse = m + log l."""
    rng = np.random.default_rng(23)
    worst = 0.0
    for causal, pad, lo, hi in [(False, 0, 5, 27), (True, 0, 4, 30), (True, 6, 0, 17)]:
        n = m = 30
        q, k, v = rnd(rng, n, 8, scale=3.0), rnd(rng, m, 8, scale=3.0), rnd(rng, m, 5)
        o, lse = oracle.attention_range(q[None, None], k[None, None], v[None, None], 0.5,
                                        causal, None if pad == 0 else [pad], lo, hi)
        mm, ll, acc = oracle.online_partial(q, np.arange(n), k, v, 0.5, 7, lo, hi, causal, pad)
        fin = ll > 0
        if not np.array_equal(fin, np.isfinite(lse[0, 0])):
            return False
        worst = max(worst, np.abs(o[0, 0] - oracle.finish(mm, ll, acc)).max(),
                    np.abs(lse[0, 0][fin] - (mm[fin] + np.log(ll[fin]))).max(initial=0.0))
    return worst <= TIGHT


# --------------------------------------------------------------------------
# paged chunked prefill: a chunk of queries at the end of each sequence
# --------------------------------------------------------------------------
def brute_force_paged_prefill(q, k_cache, v_cache, table, seq_lens, bs, scale, causal):
    """Literal loops: gather each sequence's rows through the table one token
    at a time; query row i is token L - n + i."""
    S, Hq, n, _ = q.shape
    Hkv = k_cache.shape[2]
    out = np.zeros((S, Hq, n, v_cache.shape[-1]))
    for s in range(S):
        L = int(seq_lens[s])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            ks = [k_cache[table[s, t // bs], t % bs, g] for t in range(L)]
            vs = [v_cache[table[s, t // bs], t % bs, g] for t in range(L)]
            for i in range(n):
                pos = L - n + i
                keys = [j for j in range(L) if (not causal or j <= pos)] if pos >= 0 else []
                if not keys:
                    continue
                sc = [sum(float(q[s, h, i, c]) * float(ks[j][c]) for c in range(q.shape[3])) * scale
                      for j in keys]
                w = [math.exp(x) for x in sc]
                tot = sum(w)
                for wj, j in zip(w, keys):
                    out[s, h, i] += wj / tot * vs[j]
    return out


def make_paged_chunk(rng, n, lens, S=3, Hq=4, Hkv=2, d=5, dv=6, bs=4, maxb=5):
    q1, kc, vc, table, lens, bs = make_paged(rng, S=S, Hq=Hq, Hkv=Hkv, d=d, dv=dv, bs=bs,
                                             lens=lens, maxb=maxb)
    q = rnd(rng, S, Hq, n, d)
    return q, kc, vc, table, lens, bs


def pin_paged_prefill_bruteforce():
    rng = np.random.default_rng(24)
    worst = 0.0
    for causal in (True, False):
        q, kc, vc, table, lens, bs = make_paged_chunk(rng, 5, (0, 3, 12))   # n > L for seq 1
        got = oracle.paged_prefill(q, kc, vc, table, lens, bs, 0.45, causal)
        ref = brute_force_paged_prefill(q, kc, vc, table, lens, bs, 0.45, causal)
        worst = max(worst, np.abs(got - ref).max())
    return worst <= TIGHT


def pin_paged_prefill_special_cases():
    """n = 1 is the paged decode; a chunk covering whole equal-length
    sequences is causal attention on the gathered rows."""
    rng = np.random.default_rng(25)
    q, kc, vc, table, lens, bs = make_paged_chunk(rng, 1, (1, 9, 16))
    got = oracle.paged_prefill(q, kc, vc, table, lens, bs, 0.3, True)[:, :, 0]
    dec = oracle.paged_decode(q[:, :, 0], kc, vc, table, lens, bs, 0.3)
    worst = np.abs(got - dec).max()
    L = 12
    q, kc, vc, table, lens, bs = make_paged_chunk(rng, L, (L, L), S=2)
    got = oracle.paged_prefill(q, kc, vc, table, lens, bs, 0.3, True)
    for s in range(2):
        kk = np.stack([kc[table[s, t // bs], t % bs] for t in range(L)], axis=1)  # [Hkv, L, d]
        vv = np.stack([vc[table[s, t // bs], t % bs] for t in range(L)], axis=1)
        ref = oracle.attention(q[s][None], kk[None], vv[None], 0.3, causal=True)[0]
        worst = max(worst, np.abs(got[s] - ref).max())
    return worst <= TIGHT


PINS = [pin_bruteforce_prefill, pin_bruteforce_gqa, pin_bruteforce_paged, pin_causal_row0,
        pin_causal_prefix_means, pin_hot_finite, pin_dominant_key, pin_recurrence_sweep,
        pin_split_merge,
        pin_gqa_equals_repeated_mha, pin_paged_equals_contiguous,
        pin_range_bruteforce, pin_range_merge, pin_range_matches_recurrence,
        pin_paged_prefill_bruteforce, pin_paged_prefill_special_cases]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin()


# --------------------------------------------------------------------------
# the 5688vip self-test: seed 42 (legacy generator), N = 4, d = 8, float64,
# block size 2, no scale; the tiled result must be within 1e-8 of the
# standard one
# --------------------------------------------------------------------------
def test_5688vip_worked_procedure():
    np.random.seed(42)
    Q = np.random.randn(4, 8).astype(np.float64)
    K = np.random.randn(4, 8).astype(np.float64)
    V = np.random.randn(4, 8).astype(np.float64)
    std = oracle.attention(Q[None, None], K[None, None], V[None, None], 1.0)[0, 0]
    tiled = oracle.online_attention_q_outer(Q, K, V, 1.0, q_block=2, k_block=2)
    diff = np.abs(std - tiled).max()
    assert diff < FIG["tiled_vs_standard_threshold"]["value"]
    assert diff < 1e-14
    # the standard version's P rows sum to 1
    P = oracle.probabilities(Q, K, 1.0)
    assert np.abs(P.sum(axis=1) - 1).max() < 1e-15
    # regression anchor written by tests/golden/make_golden.py (oracle only)
    golden = np.loadtxt(os.path.join(GOLDEN, "p3_seed42_output.txt"))
    assert np.abs(std - golden).max() < 1e-15


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def test_probabilities_rows_sum_to_one_and_masked_rows_zero():
    rng = np.random.default_rng(30)
    q, k = rnd(rng, 12, 8, scale=4.0), rnd(rng, 12, 8, scale=4.0)
    for causal, pad in [(False, 0), (True, 0), (True, 4)]:
        P = oracle.probabilities(q, k, 0.5, causal, pad)
        sums = P.sum(axis=1)
        assert np.abs(sums[pad:] - 1).max() < 1e-14
        assert np.all(P[:pad] == 0)
        assert np.all(P >= 0)


def test_library_softmax_special_case():
    """Non-causal P equals scipy's softmax of the scaled score matrix."""
    rng = np.random.default_rng(31)
    q, k = rnd(rng, 20, 16, scale=5.0), rnd(rng, 30, 16, scale=5.0)
    P = oracle.probabilities(q, k, 0.25)
    ref = scipy.special.softmax(0.25 * np.einsum("id,jd->ij", q, k), axis=1)
    assert np.abs(P - ref).max() < 1e-14


def test_output_within_value_range():
    rng = np.random.default_rng(32)
    q, k, v = rnd(rng, 16, 8, scale=3), rnd(rng, 16, 8, scale=3), rnd(rng, 16, 5)
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, causal=True)[0, 0]
    for i in range(16):
        lo, hi = v[:i + 1].min(axis=0), v[:i + 1].max(axis=0)
        assert np.all(o[i] >= lo - 1e-14) and np.all(o[i] <= hi + 1e-14)


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(33)
    q = rnd(rng, 7, 8)
    k = np.tile(rnd(rng, 1, 8), (10, 1))
    v = rnd(rng, 10, 4)
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 0.3)[0, 0]
    assert np.abs(o - v.mean(axis=0)).max() < TIGHT
    oc = oracle.attention(q[None, None], k[None, None, :7], v[None, None, :7], 0.3, causal=True)[0, 0]
    assert np.abs(oc - np.cumsum(v[:7], 0) / np.arange(1, 8)[:, None]).max() < TIGHT


def test_dominant_key_gives_its_value_row():
    rng = np.random.default_rng(34)
    k = rnd(rng, 12, 16)
    v = rnd(rng, 12, 6)
    j = 7
    q = (k[j] * 10.0)[None, :]          # score gap to every other key >> 50
    s = oracle.scores(q, k, 1.0)[0]
    gap = s[j] - np.delete(s, j).max()
    assert gap >= 50
    o = oracle.attention(q[None, None], k[None, None], v[None, None], 1.0)[0, 0, 0]
    assert np.abs(o - v[j]).max() < TIGHT


def test_key_value_permutation_invariance():
    rng = np.random.default_rng(35)
    q, k, v = rnd(rng, 6, 8), rnd(rng, 14, 8), rnd(rng, 14, 5)
    perm = rng.permutation(14)
    a = oracle.attention(q[None, None], k[None, None], v[None, None], 0.4)
    b = oracle.attention(q[None, None], k[None, None, perm], v[None, None, perm], 0.4)
    assert np.abs(a - b).max() < TIGHT


def test_affine_values():
    rng = np.random.default_rng(36)
    q, k, v = rnd(rng, 6, 8), rnd(rng, 9, 8), rnd(rng, 9, 5)
    a = oracle.attention(q[None, None], k[None, None], v[None, None], 0.4, causal=True)
    b = oracle.attention(q[None, None], k[None, None], (2.5 * v - 1.25)[None, None], 0.4, causal=True)
    assert np.abs(b - (2.5 * a - 1.25)).max() < TIGHT


def test_scale_moves_into_queries():
    rng = np.random.default_rng(37)
    q, k, v = rnd(rng, 6, 8), rnd(rng, 9, 8), rnd(rng, 9, 5)
    a = oracle.attention(q[None, None], k[None, None], v[None, None], 0.125)
    b = oracle.attention((0.125 * q)[None, None], k[None, None], v[None, None], 1.0)
    assert np.abs(a - b).max() < TIGHT


def test_padding_poison_never_read():
    rng = np.random.default_rng(38)
    n, pad = 10, 4
    q, k, v = rnd(rng, n, 4), rnd(rng, n, 4), rnd(rng, n, 3)
    clean = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, True, pads=[pad])
    qp, kp, vp = q.copy(), k.copy(), v.copy()
    qp[:pad] = kp[:pad] = np.nan
    vp[:pad] = np.nan
    dirty = oracle.attention(qp[None, None], kp[None, None], vp[None, None], 0.5, True, pads=[pad])
    assert np.array_equal(clean, dirty)
    assert np.all(dirty[0, 0, :pad] == 0)
    # the recurrence slices the same way
    o = oracle.online_attention(qp, kp, vp, 0.5, tile=3, causal=True, pad=pad)
    assert np.isfinite(o).all() and np.abs(o - clean[0, 0]).max() < TIGHT


def test_sampled_rows_match_full():
    rng = np.random.default_rng(39)
    B, H, n, d = 2, 3, 20, 4
    q, k, v = rnd(rng, B, H, n, d), rnd(rng, B, H, n, d), rnd(rng, B, H, n, d)
    full = oracle.attention(q, k, v, 0.5, causal=True, pads=[0, 6])
    samples = [(0, 1, 0), (1, 2, 3), (1, 0, 6), (1, 1, 19), (0, 2, 13)]
    got = oracle.attention_rows(q, k, v, 0.5, samples, causal=True, pads=[0, 6])
    for t, (b, h, i) in enumerate(samples):
        assert np.abs(got[t] - full[b, h, i]).max() < 1e-14


def test_decode_zero_length_and_chunking():
    rng = np.random.default_rng(40)
    q, kc, vc, table, lens, bs = make_paged(rng, lens=(0, 3, 12))
    o = oracle.paged_decode(q, kc, vc, table, lens, bs, 0.5)
    assert np.all(o[0] == 0)
    # row chunking of the batched definition does not change results
    q2, k2, v2 = rnd(rng, 1, 2, 50, 4), rnd(rng, 1, 2, 50, 4), rnd(rng, 1, 2, 50, 4)
    a = oracle.attention(q2, k2, v2, 0.5, True, chunk=7)
    b = oracle.attention(q2, k2, v2, 0.5, True, chunk=1024)
    assert np.abs(a - b).max() < 1e-15


# --------------------------------------------------------------------------
# negative controls: each wrong method must be detected
# --------------------------------------------------------------------------
def test_blockwise_per_block_softmax_is_wrong():
    """10100.com version 3: normalising each key block on its own and summing
    the outputs is off by O(1) (the article measured 2.1)."""
    rng = np.random.default_rng(41)
    n, m, d = 64, 256, 128
    q, k, v = rnd(rng, n, d), rnd(rng, m, d), rnd(rng, m, d)
    scale = 1 / math.sqrt(d)
    ref = oracle.attention(q[None, None], k[None, None], v[None, None], scale)[0, 0]
    outs = []
    for s in range(0, m, 16):
        p = scipy.special.softmax(scale * (q @ k[s:s + 16].T), axis=1)
        outs.append(p @ v[s:s + 16])
    v3 = np.sum(outs, axis=0)
    err = np.abs(v3 - ref).max()
    assert err > 0.5, err
    assert FIG["blockwise_bug_max_error"]["value"] / 10 < err < FIG["blockwise_bug_max_error"]["value"] * 10


def test_unsubtracted_softmax_overflows_on_hot_data():
    """10100.com section 4: with Q, K x10 the unsubtracted fp32 softmax turns
    all 512 outputs into inf/NaN; the oracle stays finite."""
    rng = np.random.default_rng(42)
    f = FIG["hot_data_factor"]["value"]
    n, m, d = 4, 256, 128
    q = (rng.standard_normal((n, d)) * f).astype(np.float32)
    k = (rng.standard_normal((m, d)) * f).astype(np.float32)
    v = rng.standard_normal((m, d)).astype(np.float32)
    scale = np.float32(1 / math.sqrt(d))
    S = (q @ k.T) * scale
    assert S.dtype == np.float32 and S.max() > 89  # past fp32 exp overflow
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(S)
        P = e / e.sum(axis=1, keepdims=True)
        O = P @ v
    assert (~np.isfinite(O)).sum() == FIG["hot_naive_nonfinite_outputs"]["value"] == O.size
    o = oracle.attention(q[None, None].astype(np.float64), k[None, None].astype(np.float64),
                         v[None, None].astype(np.float64), float(scale))
    assert np.isfinite(o).all()


def test_fp16_exp_overflow_point():
    """10100.com section 4: fp16 exp overflows past a score of about 11.1."""
    thr = FIG["fp16_exp_overflow_score"]["value"]
    assert abs(math.log(65504.0) - thr) < 0.05
    with np.errstate(over="ignore"):
        assert np.isfinite(np.exp(np.float16(11.0859375)))
        assert np.isinf(np.exp(np.float16(11.09375)))


def test_unguarded_recurrence_gives_nan_on_masked_first_tile():
    """S12: starting the running max at -inf turns a fully masked first tile
    into exp(-inf - -inf) = NaN; the finite sentinel avoids it."""
    rng = np.random.default_rng(43)
    n, d = 8, 4
    q, k, v = rnd(rng, n, d), rnd(rng, n, d), rnd(rng, n, d)
    pad = 4  # keys 0..3 are padding -> the first tile of 4 keys is fully masked
    m_run, l_run, acc = np.full(n, -np.inf), np.zeros(n), np.zeros((n, d))
    with np.errstate(invalid="ignore"):
        for j0 in range(0, n, 4):
            s = np.full((n, 4), -np.inf)
            if j0 >= pad:
                s = (q @ k[j0:j0 + 4].T) * 0.5
            m_new = np.maximum(m_run, s.max(axis=1))
            alpha = np.exp(m_run - m_new)
            p = np.exp(s - m_new[:, None])
            l_run = alpha * l_run + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[j0:j0 + 4]
            m_run = m_new
    assert np.isnan(acc).any()
    guarded = oracle.online_attention(q, k, v, 0.5, tile=4, causal=False, pad=pad)
    assert np.isfinite(guarded).all()
    ref = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, pads=[pad])[0, 0]
    assert np.abs(guarded - ref).max() < TIGHT


# --------------------------------------------------------------------------
# closed forms the pages quote
# --------------------------------------------------------------------------
def test_closed_forms():
    assert round(math.sqrt(128)) == FIG["dot_product_std_d128"]["value"]
    assert abs(32768 ** 2 * 4 - FIG["materialised_s_one_head_bytes"]["value"]) < 0.01e9
    assert abs(8192 ** 2 * 32 * 2 - 4.295e9) < 1e6
    assert 8192 ** 2 * 32 * 2 / FIG["materialised_s_8192_32heads_fp16_bytes"]["value"] < 1.1


def test_dot_product_spread_at_d128():
    rng = np.random.default_rng(44)
    a = rng.standard_normal((20000, 128))
    b = rng.standard_normal((20000, 128))
    std = np.einsum("ij,ij->i", a, b).std()
    assert abs(std - math.sqrt(128)) < 0.3


# --------------------------------------------------------------------------
# planted mistakes: every one must be caught by some pin
# --------------------------------------------------------------------------
def _scores_noscale(q, k, scale):
    return q @ k.T


def _scores_double_scale(q, k, scale):
    return (q @ k.T) * scale * scale


def _scores_sign(q, k, scale):
    return -(q @ k.T) * scale


def _allowed_strict(row_idx, key_idx, causal, pad):
    ok = np.ones((row_idx.size, key_idx.size), dtype=bool)
    if causal:
        ok &= key_idx[None, :] < row_idx[:, None]
    ok &= key_idx[None, :] >= pad
    ok &= row_idx[:, None] >= pad
    return ok


def _allowed_flipped(row_idx, key_idx, causal, pad):
    ok = np.ones((row_idx.size, key_idx.size), dtype=bool)
    if causal:
        ok &= key_idx[None, :] >= row_idx[:, None]
    ok &= key_idx[None, :] >= pad
    ok &= row_idx[:, None] >= pad
    return ok


def _allowed_no_pad_rows(row_idx, key_idx, causal, pad):
    ok = np.ones((row_idx.size, key_idx.size), dtype=bool)
    if causal:
        ok &= key_idx[None, :] <= row_idx[:, None]
    return ok


def _softmax_no_max(s, ok):
    e = np.where(ok, np.exp(np.where(ok, s, 0.0)), 0.0)
    den = e.sum(axis=1, keepdims=True)
    return np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)


def _softmax_unmasked_denominator(s, ok):
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    den = e.sum(axis=1, keepdims=True)
    return np.where(ok, e / den, 0.0)


def _gather_off_by_one(cache, table_row, seq_len, block_size, head):
    rows = []
    for logical, physical in enumerate(table_row):
        cnt = min(block_size, int(seq_len) - logical * block_size) - 1
        if cnt <= 0:
            break
        rows.append(cache[int(physical), :cnt, head])
    if not rows:
        return np.zeros((0, cache.shape[-1]))
    return np.concatenate(rows, axis=0)


def _gather_wrong_block(cache, table_row, seq_len, block_size, head):
    rows = []
    for logical, physical in enumerate(table_row):
        cnt = min(block_size, int(seq_len) - logical * block_size)
        if cnt <= 0:
            break
        rows.append(cache[logical % cache.shape[0], :cnt, head])
    return np.concatenate(rows, axis=0)


def _merge_wrong_sign(parts):
    ms = np.stack([p[0] for p in parts])
    M = ms.max(axis=0)
    l_tot = np.zeros_like(parts[0][1])
    acc_tot = np.zeros_like(parts[0][2])
    for m_s, l_s, acc_s in parts:
        w = np.exp(np.minimum(M - m_s, 50.0))
        l_tot = l_tot + w * l_s
        acc_tot = acc_tot + w[:, None] * acc_s
    return oa.finish(M, l_tot, acc_tot)


def _attention_gqa_modulo(q, k, v, scale, causal=False, pads=None, chunk=1024):
    B, Hq, n, _ = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, Hq, n, v.shape[3]))
    for b in range(B):
        pad = 0 if pads is None else int(pads[b])
        for h in range(Hq):
            out[b, h, pad:] = oa.attend(q[b, h, pad:], np.arange(pad, n), k[b, h % Hkv],
                                        v[b, h % Hkv], scale, causal, pad)
    return out


def _online_partial_no_alpha(q_rows, row_idx, k, v, scale, tile, key_lo=0, key_hi=None,
                             causal=False, pad=0):
    row_idx = np.asarray(row_idx).reshape(-1)
    key_hi = k.shape[0] if key_hi is None else key_hi
    r = q_rows.shape[0]
    m_run, l_run, acc = np.full(r, oa.SENTINEL), np.zeros(r), np.zeros((r, v.shape[1]))
    for j0 in range(key_lo, key_hi, tile):
        j1 = min(key_hi, j0 + tile)
        lo = max(j0, pad)
        s = np.full((r, j1 - j0), -np.inf)
        if lo < j1:
            s[:, lo - j0:] = oa.scores(q_rows, k[lo:j1], scale)
        s = np.where(oa.allowed_keys(row_idx, np.arange(j0, j1), causal, pad), s, -np.inf)
        m_new = np.maximum(m_run, s.max(axis=1))
        alpha = np.exp(m_run - m_new)
        p = np.exp(s - m_new[:, None])
        l_run = alpha * l_run + p.sum(axis=1)
        vt = np.zeros((j1 - j0, v.shape[1]))
        if lo < j1:
            vt[lo - j0:] = v[lo:j1]
        acc = acc + p @ vt                     # forgot to rescale the history
        m_run = m_new
    return m_run, l_run, acc


def _range_ignores_begin(q, k, v, scale, causal=False, pads=None, key_begin=0, key_end=None):
    return oa_attention_range(q, k, v, scale, causal, pads, 0, key_end)


def _range_lse_without_max(q, k, v, scale, causal=False, pads=None, key_begin=0, key_end=None):
    o, lse = oa_attention_range(q, k, v, scale, causal, pads, key_begin, key_end)
    # forgets to add the max back: log(sum exp(s - max)) only
    B, Hq, n, _ = q.shape
    group = Hq // k.shape[1]
    ke = k.shape[2] if key_end is None else key_end
    for b in range(B):
        pad = 0 if pads is None else int(pads[b])
        lo = max(key_begin, pad)
        if lo >= ke:
            continue
        for h in range(Hq):
            s = oa.scores(q[b, h], k[b, h // group, lo:ke], scale)
            ok = oa.allowed_keys(np.arange(n), np.arange(lo, ke), causal, pad)
            mx = np.where(ok, s, -np.inf).max(axis=1)
            lse[b, h] = np.where(np.isfinite(mx), lse[b, h] - np.where(np.isfinite(mx), mx, 0), -np.inf)
    return o, lse


def _merge_lse_wrong_sign(parts):
    flipped = [(o_s, np.where(np.isfinite(l_s), -l_s, l_s)) for o_s, l_s in parts]
    return oa_merge_lse(flipped)


def _paged_prefill_top_left(q, k_cache, v_cache, block_table, seq_lens, block_size, scale,
                            causal=True):
    """Chunk rows placed at positions 0 .. n-1 instead of the end."""
    S, Hq, n, _ = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    out = np.zeros((S, Hq, n, v_cache.shape[-1]))
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        for g in range(Hkv):
            kg = oa.gather_paged(k_cache, block_table[s], L, block_size, g)
            vg = oa.gather_paged(v_cache, block_table[s], L, block_size, g)
            for h in range(g * group, (g + 1) * group):
                out[s, h] = oa.attend(q[s, h], np.arange(n), kg, vg, scale, causal)
    return out


oa_attention_range = oa.attention_range
oa_merge_lse = oa.merge_lse

MUTANTS = {
    "paged_prefill_top_left": ("paged_prefill", _paged_prefill_top_left),
    "range_ignores_key_begin": ("attention_range", _range_ignores_begin),
    "range_lse_without_max": ("attention_range", _range_lse_without_max),
    "merge_lse_wrong_sign": ("merge_lse", _merge_lse_wrong_sign),
    "scores_without_scale": ("scores", _scores_noscale),
    "scores_scaled_twice": ("scores", _scores_double_scale),
    "scores_wrong_sign": ("scores", _scores_sign),
    "causal_strict": ("allowed_keys", _allowed_strict),
    "causal_flipped": ("allowed_keys", _allowed_flipped),
    "padding_rows_not_masked": ("allowed_keys", _allowed_no_pad_rows),
    "softmax_without_max": ("masked_softmax", _softmax_no_max),
    "softmax_masked_in_denominator": ("masked_softmax", _softmax_unmasked_denominator),
    "paged_gather_off_by_one": ("gather_paged", _gather_off_by_one),
    "paged_gather_ignores_table": ("gather_paged", _gather_wrong_block),
    "merge_wrong_sign": ("merge_partials", _merge_wrong_sign),
    "gqa_modulo_mapping": ("attention", _attention_gqa_modulo),
    "recurrence_without_rescale": ("online_partial", _online_partial_no_alpha),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    monkeypatch.setattr(oracle, attr, fn, raising=False)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                passed = pin()
        except Exception:
            passed = False
        if not passed:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
