"""Error bound of the FP8 attention path against the float64 definition.

The FP8 kernel differs from exact arithmetic in four places, each bounded
here in units where the largest weight of a row is 1 (pm_j = exp(s_j - max s)):

1. scores are sums of exact code products in the matrix cores, whose internal
   adders keep about 13 bits below the largest product of a group (measured on
   gfx950: worst error 1.1e-4 = 2^-13.1 of sum |products| on random E4M3
   operands spanning every exponent; 65536 + 1 - 65536 in one group gives 0).
   The bound takes ds_j = 2^-12 of scale * sum_t |q_t k_t|, so the weight
   before rounding is w_j = pm_j exp(+-ds_j).  On "hot" inputs (scores of
   several hundred) this term outweighs the E4M3 rounding of the weights;
2. the weights enter the P.V product rounded to E4M3.  The kernel's weights
   are w_j times 2^(max - m_run) >= 1 (the running max never exceeds the true
   max).  In the normal range a weight moves by at most 2^-4 of itself; below
   the smallest normal (2^-6) the spacing is 2^-9, so it moves by at most
   2^-10, and never by more than itself (it may round to 0).  In pm units:
   e_j = pm_j (exp(ds_j)(1 + 2^-4) - 1) + [pm_j exp(-ds_j) < 2^-6] min(2^-10,
   pm_j exp(ds_j));
3. the P.V and l sums carry the same 2^-12 relative to sum_j |p_j v_j|;
4. the output is rounded (bfloat16 half-ulp 2^-9) after an fp32 epilogue:
   2^-8 |O| covers both.

With e_j the bound of |p~_j - pm_j|, the error of a weighted mean
O = sum p~ v / sum p~ is sum_j (p~_j - pm_j)(v_j - O) / sum p~, so

  |err_ic| <= [sum_j e_j |v_jc - O_ic| + 2^-12 sum_j (pm_j + e_j)|v_jc|]
              / (sum_j pm_j - sum_j e_j) + 2^-8 |O_ic|          (rigorous)

and, the rounding errors being zero-mean and independent across keys,

  E[err_ic^2] <= sum_j e_j^2 (v_jc - O_ic)^2 / (sum pm - sum e)^2 + (2^-9 O_ic)^2.

The tests hold every element to the first and the root-mean-square error to
twice the square root of the mean of the second.
"""
import numpy as np

import oracle

REL_P = 2.0 ** -4
ABS_P = 2.0 ** -10
SUB_P = 2.0 ** -6
MFMA_REL = 2.0 ** -12
OUT_REL = 2.0 ** -8


def row_bounds(q_rows, row_idx, k, v, scale, causal=False, pad=0):
    """For query rows q_rows [r, d] at positions row_idx of one head with keys
    k [m, d] and values v [m, dv] (real float64 values): the oracle output
    O [r, dv], the rigorous bound B [r, dv] and the rms estimate sig [r, dv]."""
    row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
    key_idx = np.arange(k.shape[0], dtype=np.int64)
    ok = oracle.allowed_keys(row_idx, key_idx, causal, pad)
    P = oracle.masked_softmax(oracle.scores(q_rows, k, scale), ok)
    O = P @ v
    top = P.max(axis=1, keepdims=True)
    has = top[:, 0] > 0
    pm = P / np.where(top > 0, top, 1.0)
    ds = MFMA_REL * scale * (np.abs(q_rows) @ np.abs(k).T)
    grow = np.exp(ds)
    sub = (pm / grow < SUB_P) & ok
    e = pm * (grow * (1.0 + REL_P) - 1.0) + np.where(sub, np.minimum(ABS_P, pm * grow), 0.0)
    den = pm.sum(axis=1) - e.sum(axis=1)
    B = np.zeros_like(O)
    sig = np.zeros_like(O)
    av = np.abs(v)
    for i in np.nonzero(has)[0]:
        dev = np.abs(v - O[i])                     # [m, dv]
        num = e[i] @ dev + MFMA_REL * ((pm[i] + e[i]) @ av)
        B[i] = num / den[i] + OUT_REL * np.abs(O[i])
        sig[i] = np.sqrt((e[i] ** 2) @ dev ** 2) / den[i]
        sig[i] = np.sqrt(sig[i] ** 2 + (2.0 ** -9 * O[i]) ** 2)
    assert np.all(den[has] > 0), "bound undefined: rounding could cancel a row's weights"
    return O, B, sig


def row_bounds_fast(q_rows, row_idx, k, v, scale, causal=False, pad=0):
    """row_bounds in matrix products only, for whole outputs.  The rms
    estimate is the same: sum_j e_j^2 (v_j - O)^2 expands into
    (e^2) v^2 - 2 O (e^2) v + O^2 sum e^2.  The rigorous bound takes
    sum_j e_j |v_j - O| <= sqrt(sum_j e_j) sqrt(sum_j e_j (v_j - O)^2)
    (Cauchy-Schwarz, e_j >= 0) in place of the per-row sum, so it is never
    tighter than row_bounds' and still holds wherever that one does."""
    row_idx = np.asarray(row_idx, dtype=np.int64).reshape(-1)
    key_idx = np.arange(k.shape[0], dtype=np.int64)
    ok = oracle.allowed_keys(row_idx, key_idx, causal, pad)
    P = oracle.masked_softmax(oracle.scores(q_rows, k, scale), ok)
    O = P @ v
    top = P.max(axis=1, keepdims=True)
    has = top[:, 0] > 0
    pm = P / np.where(top > 0, top, 1.0)
    ds = MFMA_REL * scale * (np.abs(q_rows) @ np.abs(k).T)
    grow = np.exp(ds)
    sub = (pm / grow < SUB_P) & ok
    e = pm * (grow * (1.0 + REL_P) - 1.0) + np.where(sub, np.minimum(ABS_P, pm * grow), 0.0)
    den = pm.sum(axis=1) - e.sum(axis=1)
    assert np.all(den[has] > 0), "bound undefined: rounding could cancel a row's weights"
    den = np.where(has, den, 1.0)[:, None]
    v2 = v * v

    def dev2(w):  # sum_j w_j (v_j - O)^2, per row and column
        return np.maximum(w @ v2 - 2.0 * O * (w @ v) + O * O * w.sum(axis=1, keepdims=True), 0.0)

    num = np.sqrt(e.sum(axis=1, keepdims=True) * dev2(e)) + MFMA_REL * ((pm + e) @ np.abs(v))
    B = np.where(has[:, None], num / den + OUT_REL * np.abs(O), 0.0)
    sig = np.sqrt(dev2(e * e)) / den
    sig = np.where(has[:, None], np.sqrt(sig ** 2 + (2.0 ** -9 * O) ** 2), 0.0)
    return O, B, sig


def head_bounds(q, k, v, scale, causal=False, pad=0, chunk=128):
    """row_bounds over all rows of one head (rows before pad get zeros)."""
    n = q.shape[0]
    O = np.zeros((n, v.shape[1]))
    B = np.zeros_like(O)
    sig = np.zeros_like(O)
    ks, vs = k[pad:], v[pad:]
    for r0 in range(pad, n, chunk):
        r1 = min(n, r0 + chunk)
        o, b, s = row_bounds(q[r0:r1], np.arange(r0, r1) - pad, ks, vs, scale, causal, 0)
        O[r0:r1], B[r0:r1], sig[r0:r1] = o, b, s
    return O, B, sig


def check(got, ref, B, sig, label, say=print):
    """Element bound and rms bound; returns (max err/B, rms err / rms sig)."""
    assert np.all(np.isfinite(got)), f"{label}: non-finite outputs"
    err = np.abs(got - ref)
    ratio = float(np.max(np.where(B > 0, err / np.where(B > 0, B, 1), np.where(err > 0, np.inf, 0))))
    rms = float(np.sqrt(np.mean(err ** 2)))
    rms_sig = float(np.sqrt(np.mean(sig ** 2)))
    say(f"  {label}: max_abs={err.max():.3e} worst err/bound={ratio:.3f} "
        f"rms={rms:.3e} rms_sigma={rms_sig:.3e}")
    assert ratio <= 1.0, f"{label}: error above the FP8 bound (worst ratio {ratio:.3f})"
    assert rms <= 2.0 * rms_sig, f"{label}: rms error {rms:.3e} above 2 x {rms_sig:.3e}"
    return ratio, rms / max(rms_sig, 1e-300)
