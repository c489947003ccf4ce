"""GPU parity of the key-range path: ``fa_fwd_partial`` (attention over keys in
[key_begin, key_end) with its log-sum-exp) and ``fa_merge`` (the rescale that
joins pieces of disjoint key ranges), against the float64 oracle's
``attention_range`` / ``merge_lse`` / ``attention`` on the same seeded inputs.

Bars: the output of a piece and of a merge meets the fa_fwd bar for the input
dtype (max abs <= 1e-2 and mean abs <= 1e-3 for 16-bit inputs, 1e-5 for
float32).  lse has no bar of its own in the pages; it is ln of a sum of
weights that the kernels round to the input type (relative error below 2^-8),
plus fp32 score rounding, so 16-bit inputs get |lse error| <= 1e-2 and float32
inputs 1e-5, each plus two float32 ulps of |lse| because lse is stored as
float32 (hot rows reach |lse| of several hundred, where an ulp is 3e-5).
Rows without keys must give o = 0 and lse = -inf exactly."""
import zlib

import numpy as np
import pytest

import oracle
from tiled_online_softmax_04_amd import fa
from tiled_online_softmax_04_amd import inputs as gen

from gpu_util import assert_whole, error_sums, pooled, assert_parity, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-5, "f16": 1e-2, "bf16": 1e-2}


def dev_inputs(x, dtype):
    import torch
    q, k, v = to_dev(x["q"], dtype), to_dev(x["k"], dtype), to_dev(x["v"], dtype)
    sl = None if x["seq_lens"] is None else torch.from_numpy(x["seq_lens"]).cuda()
    return q, k, v, sl


def check_lse(got, ref, dtype, label):
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), f"{label}: -inf pattern differs"
    fin = ~inf_ref
    assert np.all(np.isfinite(got[fin])), f"{label}: non-finite lse"
    err = np.abs(got[fin] - ref[fin])
    bound = LSE_TOL[dtype] + 2.0 ** -22 * np.abs(ref[fin])
    say(f"  {label}: lse max_abs={float(err.max(initial=0.0)):.3e} "
        f"worst err/bound={float((err / bound).max(initial=0.0)):.3f}")
    assert np.all(err <= bound), f"{label}: lse error above {LSE_TOL[dtype]} + 2 ulp(|lse|)"


CASES = [
    # name, dtype, B, Hq, Hkv, n, m, d, causal, hot, lens, ranges
    ("bf16_noncausal", "bf16", 2, 4, 4, 300, 300, 128, False, 1.0, None,
     [(0, 300), (37, 211), (150, 150), (0, 5), (299, 300)]),
    ("bf16_causal", "bf16", 1, 3, 3, 333, 333, 128, True, 1.0, None,
     [(0, 333), (64, 128), (100, 333), (0, 1)]),
    ("f16_causal_hot", "f16", 1, 2, 2, 520, 520, 128, True, 10.0, None, [(0, 260), (260, 520)]),
    ("bf16_causal_leftpad", "bf16", 4, 2, 2, 400, 400, 128, True, 1.0, [400, 1, 0, 137],
     [(0, 200), (200, 400), (250, 399)]),
    ("bf16_gqa_d64", "bf16", 1, 8, 2, 200, 200, 64, True, 1.0, None, [(13, 190)]),
    ("f16_n_ne_m", "f16", 2, 2, 1, 100, 333, 128, False, 1.0, None, [(0, 100), (100, 333)]),
    ("f32_causal_leftpad_hot", "f32", 2, 2, 2, 100, 100, 64, True, 10.0, [100, 33],
     [(0, 50), (50, 100), (7, 93)]),
    ("f32_gqa_d128", "f32", 1, 4, 2, 77, 77, 128, False, 1.0, None, [(10, 60)]),
]


def make(case):
    name, dtype, B, Hq, Hkv, n, m, d, causal, hot, lens, ranges = case
    x = gen.make_prefill_custom(dtype, B, Hq, Hkv, n, m, d, d,
                                seed=zlib.crc32(name.encode()) % 1000, hot=hot, lens=lens)
    return x, float(np.float32(1 / np.sqrt(d)))


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_partial_pieces(case):
    import torch
    name, dtype, causal, ranges = case[0], case[1], case[8], case[11]
    say(f"[key-range] {name}")
    x, scale = make(case)
    q, k, v, sl = dev_inputs(x, dtype)
    qf, kf, vf = (gen.to_f64(x[t], dtype) for t in ("q", "k", "v"))
    for lo, hi in ranges:
        o, lse = fa.fwd_partial(q, k, v, lo, hi, scale=scale, causal=causal, seq_lens=sl)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attention_range(qf, kf, vf, scale, causal, x["pads"], lo, hi)
        got_o, got_l = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        assert_parity(got_o, ref_o, dtype, f"{name} [{lo},{hi}) o")
        check_lse(got_l, ref_l, dtype, f"{name} [{lo},{hi})")
        none = np.isneginf(ref_l)
        assert np.all(got_o[none] == 0), "rows without keys must give o = 0"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_merge_reproduces_full_pass(case):
    import torch
    name, dtype, B, Hq, n, m, causal = case[0], case[1], case[2], case[3], case[5], case[6], case[8]
    say(f"[key-range merge] {name}")
    x, scale = make(case)
    q, k, v, sl = dev_inputs(x, dtype)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    cuts = np.sort(rng.integers(0, m + 1, size=2))
    bounds = [0, *cuts.tolist(), m]                 # three ranges, possibly empty ones
    pieces = [fa.fwd_partial(q, k, v, lo, hi, scale=scale, causal=causal, seq_lens=sl)
              for lo, hi in zip(bounds[:-1], bounds[1:])]
    o_parts = torch.stack([p[0] for p in pieces])
    l_parts = torch.stack([p[1] for p in pieces])
    out, lse = fa.merge(o_parts, l_parts, out_dtype=q.dtype, want_lse=True)
    full = fa.fwd(q, k, v, scale=scale, causal=causal, seq_lens=sl)
    torch.cuda.synchronize()
    qf, kf, vf = (gen.to_f64(x[t], dtype) for t in ("q", "k", "v"))
    ref = oracle.attention(qf, kf, vf, scale, causal, pads=x["pads"])
    _, ref_l = oracle.attention_range(qf, kf, vf, scale, causal, x["pads"])
    got = to_f64(out, dtype)
    assert_parity(got, ref, dtype, f"{name} bounds={bounds} merged")
    assert_parity(got, to_f64(full, dtype), dtype, f"{name} merged vs single pass")
    check_lse(lse.cpu().numpy().astype(np.float64), ref_l, dtype, f"{name} merged")
    if x["pads"] is not None:
        for b, p in enumerate(x["pads"]):
            assert np.all(got[b, :, :p] == 0)


def _random_cases():
    rng = np.random.default_rng(20261206)
    out = []
    for i in range(12):
        dtype = ["bf16", "f16"][int(rng.integers(2))]
        d = [64, 128][int(rng.integers(2))]
        B = int(rng.integers(1, 4))
        Hkv = [1, 2, 4][int(rng.integers(3))]
        Hq = Hkv * [1, 2, 4][int(rng.integers(3))]
        causal = bool(rng.integers(2))
        n = int(rng.integers(1, 700))
        ragged = rng.random() < 0.3
        m = n if (causal or ragged) else int(rng.integers(1, 700))
        lens = [int(x) for x in rng.integers(0, n + 1, size=B)] if ragged else None
        cuts = np.sort(rng.integers(0, m + 1, size=int(rng.integers(0, 4)))).tolist()
        bounds = [0, *cuts, m]
        out.append((f"r{i:02d}_{dtype}_d{d}_B{B}_H{Hq}x{Hkv}_n{n}_m{m}"
                    f"{'_causal' if causal else ''}{'_pad' if ragged else ''}_{len(bounds) - 1}pieces",
                    dtype, B, Hq, Hkv, n, m, d, causal, 1.0, lens,
                    list(zip(bounds[:-1], bounds[1:]))))
    return out


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_partition(case):
    """Seeded random shapes, each cut into 1-4 key ranges (empty ones
    included): every piece's o and lse against the oracle's attention_range,
    and their merge against the definition."""
    import torch
    name, dtype, causal, ranges = case[0], case[1], case[8], case[11]
    say(f"[key-range random] {name} {ranges}")
    x, scale = make(case)
    q, k, v, sl = dev_inputs(x, dtype)
    qf, kf, vf = (gen.to_f64(x[t], dtype) for t in ("q", "k", "v"))
    pieces = []
    for lo, hi in ranges:
        o, lse = fa.fwd_partial(q, k, v, lo, hi, scale=scale, causal=causal, seq_lens=sl)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.attention_range(qf, kf, vf, scale, causal, x["pads"], lo, hi)
        got_o, got_l = o.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        assert_parity(got_o, ref_o, dtype, f"{name} [{lo},{hi}) o")
        check_lse(got_l, ref_l, dtype, f"{name} [{lo},{hi})")
        assert np.all(got_o[np.isneginf(ref_l)] == 0), "rows without keys must give o = 0"
        pieces.append((o, lse))
    out = fa.merge(torch.stack([p_[0] for p_ in pieces]), torch.stack([p_[1] for p_ in pieces]),
                   out_dtype=q.dtype)
    torch.cuda.synchronize()
    ref = oracle.attention(qf, kf, vf, scale, causal, pads=x["pads"])
    assert_parity(to_f64(out, dtype), ref, dtype, f"{name} merged")


@pytest.mark.parametrize("bounds", [[0, 17, 17, 40, 64], [0, 9, 17, 17, 30, 40, 64]],
                         ids=["4pieces", "6pieces"])
def test_merge_kernel_on_oracle_pieces(bounds):
    """The merge alone: pieces computed by the oracle (float32), merged on the
    GPU, against the oracle's merge_lse; includes rows covered by no piece.
    The o of a piece without keys (lse = -inf) is never read: poisoning it
    with NaN leaves the result bitwise unchanged."""
    import torch
    rng = np.random.default_rng(31)
    B, Hq, n, m, d = 2, 3, 50, 64, 64
    q, k, v = (rng.standard_normal(s) for s in [(B, Hq, n, d), (B, Hq, m, d), (B, Hq, m, d)])
    pads = [0, 20]
    parts = [oracle.attention_range(q, k, v, 0.125, True, pads, lo, hi)
             for lo, hi in zip(bounds[:-1], bounds[1:])]
    o32 = [p_[0].astype(np.float32) for p_ in parts]
    l32 = [p_[1].astype(np.float32) for p_ in parts]
    ref_o, ref_l = oracle.merge_lse([(a.astype(np.float64), b.astype(np.float64))
                                     for a, b in zip(o32, l32)])
    o_parts = torch.from_numpy(np.stack(o32)).cuda()
    l_parts = torch.from_numpy(np.stack(l32)).cuda()
    for dt, label in [(torch.float32, "f32")]:
        out, lse = fa.merge(o_parts, l_parts, out_dtype=dt, want_lse=True)
        torch.cuda.synchronize()
        assert_parity(out.cpu().numpy().astype(np.float64), ref_o, label, "merge of oracle pieces")
        check_lse(lse.cpu().numpy().astype(np.float64), ref_l, label, "merge of oracle pieces")
    out16 = fa.merge(o_parts, l_parts, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(to_f64(out16, "bf16"), ref_o, "bf16", "merge of oracle pieces, bf16 out")
    empty = torch.isinf(l_parts) & (l_parts < 0)
    assert bool(empty.any())
    poisoned = o_parts.clone()
    poisoned[empty] = float("nan")
    out_p, lse_p = fa.merge(poisoned, l_parts, out_dtype=torch.float32, want_lse=True)
    out_c, lse_c = fa.merge(o_parts, l_parts, out_dtype=torch.float32, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)


def test_full_size_key_split_whole_output():
    """The bf16 2048-key workload split into four 512-key ranges in the launch
    the benchmark times: every piece's fp32 o and its lse against the oracle's
    attention_range, and every element of the merged output against the
    definition; the merged result also against fa_fwd."""
    import torch
    w = gen.WORKLOADS["bf16_b4_2048"]
    say("[key-range] bf16_b4_2048 in four key ranges")
    x = gen.make_prefill(w)
    q, k, v, _ = dev_inputs(x, w.dtype)
    bounds = [0, 512, 1024, 1536, 2048]
    pieces = [fa.fwd_partial(q, k, v, lo, hi, scale=w.scale) for lo, hi in zip(bounds[:-1],
                                                                               bounds[1:])]
    o_parts = torch.stack([p[0] for p in pieces])
    l_parts = torch.stack([p[1] for p in pieces])
    out = fa.merge(o_parts, l_parts, out_dtype=q.dtype)
    full = fa.fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    diff = (out.float() - full.float()).abs()
    say(f"  merged vs single pass: max={diff.max().item():.3e} mean={diff.mean().item():.3e}")
    assert diff.max().item() <= 1e-2 and diff.mean().item() <= 1e-3
    got_o = o_parts.cpu().numpy()
    got_l = l_parts.cpu().numpy()
    got_m = out.view(torch.int16).cpu().numpy().view(np.uint16)
    del o_parts, l_parts, out, full, pieces
    g = w.Hq // w.Hkv

    def one(bh):
        b, h = bh
        qh = gen.to_f64(x["q"][b, h], w.dtype)[None, None]
        kh = gen.to_f64(x["k"][b, h // g], w.dtype)[None, None]
        vh = gen.to_f64(x["v"][b, h // g], w.dtype)[None, None]
        piece_errs, lse_ratio = [], 0.0
        for i, (lo, hi) in enumerate(zip(bounds[:-1], bounds[1:])):
            ro, rl = oracle.attention_range(qh, kh, vh, w.scale, False, None, lo, hi)
            piece_errs.append(error_sums(got_o[i, b, h].astype(np.float64), ro[0, 0]))
            err = np.abs(got_l[i, b, h].astype(np.float64) - rl[0, 0])
            lse_ratio = max(lse_ratio, float(np.max(err / (LSE_TOL[w.dtype] +
                                                           2.0 ** -22 * np.abs(rl[0, 0])))))
        ref = oracle.attention(qh, kh, vh, w.scale, False)[0, 0]
        merged = error_sums(gen.bf16_bits_to_f64(got_m[b, h]), ref)
        return piece_errs, lse_ratio, merged

    res = pooled(one, [(b, h) for b in range(w.B) for h in range(w.Hq)])
    assert_whole([p for r in res for p in r[0]], w.dtype, "bf16_b4_2048 key pieces (fp32 o)")
    worst = max(r[1] for r in res)
    say(f"  bf16_b4_2048 key pieces: worst lse error / bar = {worst:.3f}")
    assert worst <= 1.0
    assert_whole([r[2] for r in res], w.dtype, "bf16_b4_2048 key split, merged")
