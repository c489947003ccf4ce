"""FP8 inputs for the float64 attention oracle.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: nothing on the product
path imports it.  It shares no code with the HIP library.

The pages mention FP8 only as a capability that FlashAttention-3 added on
Hopper (llminference.xinbetween.com S12, the production list "在生产环境中").
They fix neither the format nor how scales enter, so this follows the plainest
reading:

* storage is OCP 8-bit floating point, E4M3 variant ("e4m3fn": 1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits, no infinities, the all-ones
  exponent-and-mantissa code is NaN, largest finite value 448), which is the
  FP8 format CDNA4 matrix cores read;
* each of Q, K, V carries one float32 "descale" factor: the real input is
  descale * decode(code);
* the attention computed is the plain definition (``sdpa.attention``) on those
  real inputs, in float64.
"""
from __future__ import annotations

import numpy as np

from . import sdpa

E4M3_BIAS = 7


def e4m3_to_f64(codes) -> np.ndarray:
    """Exact float64 value of each E4M3 code (uint8 array).

    exponent field e and mantissa field f: e > 0 gives (1 + f/8) * 2^(e - 7),
    e == 0 gives (f/8) * 2^(1 - 7) (subnormals, and zero); codes 0x7F and 0xFF
    are NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + f / 8.0, (e - E4M3_BIAS).astype(np.int64))
    sub = np.ldexp(f / 8.0, 1 - E4M3_BIAS)
    val = sign * np.where(e > 0, normal, sub)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def dequantize(codes, descale: float) -> np.ndarray:
    """descale * decode(codes), with descale taken as the float32 the kernel
    receives, converted exactly to float64."""
    return e4m3_to_f64(codes) * float(np.float32(descale))


def attention_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                  scale: float, causal: bool = False, pads=None) -> np.ndarray:
    """O [B, Hq, n, dv] of the plain definition on the dequantized inputs
    (shapes as ``sdpa.attention``).  Padding rows may hold NaN codes: the
    definition never reads them."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    return sdpa.attention(q, k, v, scale, causal, pads)
