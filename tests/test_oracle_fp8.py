"""Pins for the FP8 (E4M3) part of the oracle (CPU only).

The decoder is tied to the format's definition (closed-form codes) and to a
library routine (torch's float8_e4m3fn cast, all 256 codes); the attention on
dequantized inputs is tied to a brute-force loop that decodes every code by
hand, and to two scale invariants.  Planted mistakes must fail a pin."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as of

TIGHT = 1e-12


def decode_by_hand(code: int) -> float:
    """One E4M3 code, field by field (sign, 4-bit exponent with bias 7, 3-bit
    mantissa; exponent 0 is subnormal; S.1111.111 is NaN)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    f = code & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(f, -9)
    return s * math.ldexp(8 + f, e - 10)


def brute_force_fp8(q8, k8, v8, qd, kd, vd, scale, causal, pads):
    B, Hq, n, d = q8.shape
    Hkv, m, dv = k8.shape[1], k8.shape[2], v8.shape[3]
    g = Hq // Hkv
    qd, kd, vd = (float(np.float32(x)) for x in (qd, kd, vd))
    out = np.zeros((B, Hq, n, dv))
    for b in range(B):
        pad = 0 if pads is None else int(pads[b])
        for h in range(Hq):
            for i in range(pad, n):
                keys = [j for j in range(pad, m) if not (causal and j > i)]
                if not keys:
                    continue
                s = []
                for j in keys:
                    acc = 0.0
                    for t in range(d):
                        acc += (qd * decode_by_hand(int(q8[b, h, i, t]))) * \
                               (kd * decode_by_hand(int(k8[b, h // g, j, t])))
                    s.append(acc * scale)
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                for c in range(dv):
                    out[b, h, i, c] = sum(wj * vd * decode_by_hand(int(v8[b, h // g, j, c]))
                                          for wj, j in zip(w, keys)) / tot
    return out


def rand_codes(rng, shape):
    """Random finite E4M3 codes (every exponent, subnormals included)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] ^= 0x01          # 0x7F -> 0x7E (448), 0xFF -> 0xFE
    return c


def pin_decoder_closed_forms():
    want = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
            0x30: 0.5, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
            0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    got = oracle.e4m3_to_f64(np.array(list(want), dtype=np.uint8))
    if not np.array_equal(got, np.array(list(want.values()))):
        return False
    if not (np.isnan(oracle.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()):
        return False
    pos = oracle.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    return bool(np.all(np.diff(pos) > 0) and np.signbit(oracle.e4m3_to_f64(np.uint8(0x80))))


def pin_decoder_matches_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    return bool(np.array_equal(np.isnan(ours), np.isnan(lib)) and
                np.array_equal(ours[~np.isnan(ours)], lib[~np.isnan(lib)]))


def pin_decoder_matches_hand():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    hand = np.array([decode_by_hand(int(c)) for c in codes])
    return bool(np.array_equal(np.nan_to_num(ours, nan=7e7), np.nan_to_num(hand, nan=7e7)))


def pin_attention_bruteforce():
    rng = np.random.default_rng(8)
    ok = True
    for causal, pads in ((False, None), (True, None), (True, [0, 2]), (False, [3, 0])):
        q8 = rand_codes(rng, (2, 4, 5, 3))
        k8 = rand_codes(rng, (2, 2, 5, 3))
        v8 = rand_codes(rng, (2, 2, 5, 2))
        # descales that bring the codes' wide range to moderate scores
        qd, kd, vd = 1.0 / 96, 1.0 / 160, 0.01
        got = oracle.attention_fp8(q8, k8, v8, qd, kd, vd, 0.5, causal, pads)
        ref = brute_force_fp8(q8, k8, v8, qd, kd, vd, 0.5, causal, pads)
        scale_v = np.abs(oracle.e4m3_to_f64(v8)).max() * vd
        ok &= bool(np.abs(got - ref).max() <= TIGHT * max(scale_v, 1.0))
    return ok


def pin_descale_invariants():
    rng = np.random.default_rng(9)
    q8 = rand_codes(rng, (1, 2, 6, 4))
    k8 = rand_codes(rng, (1, 2, 6, 4))
    v8 = rand_codes(rng, (1, 2, 6, 4))
    base = oracle.attention_fp8(q8, k8, v8, 0.01, 0.02, 0.5, 0.25, True)
    # a factor 2 moved from K's descale to Q's leaves every score unchanged
    moved = oracle.attention_fp8(q8, k8, v8, 0.02, 0.01, 0.5, 0.25, True)
    # doubling V's descale doubles O
    doubled = oracle.attention_fp8(q8, k8, v8, 0.01, 0.02, 1.0, 0.25, True)
    # K's descale acts as a temperature: K descale 0 gives the prefix means
    flat = oracle.attention_fp8(q8, k8, v8, 0.01, 0.0, 0.5, 0.25, True)
    vv = oracle.e4m3_to_f64(v8) * 0.5
    prefix = np.cumsum(vv, axis=2) / np.arange(1, 7)[None, None, :, None]
    return bool(np.array_equal(base, moved) and np.array_equal(doubled, 2 * base) and
                np.abs(flat - prefix).max() <= TIGHT)


PINS = [pin_decoder_closed_forms, pin_decoder_matches_library, pin_decoder_matches_hand,
        pin_attention_bruteforce, pin_descale_invariants]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin()


# planted mistakes ------------------------------------------------------------
def _decode_bias8(codes):
    return of.__wrapped_decode(codes) * 0.5


def _decode_flush_subnormals(codes):
    v = of.__wrapped_decode(codes)
    c = np.asarray(codes, dtype=np.uint8)
    return np.where((c & 0x78) == 0, 0.0 * v, v)


def _decode_mantissa_16(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = of.__wrapped_decode(codes)
    e = (c >> 3) & 0xF
    f = (c & 7).astype(np.float64)
    return np.where(e > 0, np.sign(v) * np.ldexp(1.0 + f / 16.0, e - 7), v)


def _attention_ignores_k_descale(q8, k8, v8, q_descale, k_descale, v_descale, scale,
                                 causal=False, pads=None):
    return of.__wrapped_attention(q8, k8, v8, q_descale, 1.0, v_descale, scale, causal, pads)


def _attention_v_descale_squared(q8, k8, v8, q_descale, k_descale, v_descale, scale,
                                 causal=False, pads=None):
    return of.__wrapped_attention(q8, k8, v8, q_descale, k_descale, v_descale ** 2, scale,
                                  causal, pads)


MUTANTS = {
    "decode_bias_8": ("e4m3_to_f64", _decode_bias8),
    "decode_flushes_subnormals": ("e4m3_to_f64", _decode_flush_subnormals),
    "decode_mantissa_over_16": ("e4m3_to_f64", _decode_mantissa_16),
    "attention_ignores_k_descale": ("attention_fp8", _attention_ignores_k_descale),
    "attention_v_descale_squared": ("attention_fp8", _attention_v_descale_squared),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(of, "__wrapped_decode", of.e4m3_to_f64, raising=False)
    monkeypatch.setattr(of, "__wrapped_attention", of.attention_fp8, raising=False)
    monkeypatch.setattr(of, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
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
