"""Seeded synthetic inputs for the attention workloads.

This module is shared by the tests, the benchmark and the oracle checks.  It
draws random numbers and rounds them to the storage dtypes; it contains none
of the attention arithmetic (no scores, no softmax, no weighted sums).

Recipe (every workload):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * draws, in this order: Q, K, V as float32 standard normals, then the
    ragged lengths / sequence lengths (integers, inclusive bounds), then the
    physical block permutation of a paged cache;
  * "hot" data multiplies Q and K by 10 in float32 before the cast (the
    overflow experiment of the 10100.com article, section 4);
  * storage casts are round-to-nearest-even: float32 -> bfloat16 by bit
    arithmetic, float32 -> float16 by numpy's cast.
  * FP8 ("fp8": OCP E4M3, the e4m3fn encoding) is stored per tensor: the
    float32 draws are divided by descale = amax / 448 (a float32) and rounded
    to nearest-even E4M3 codes (uint8); the descale travels with the codes.
Padding rows of a left-padded batch, cache slots past a sequence's length and
unused block-table columns hold poison (NaN / -1) so that a kernel that reads
them is caught.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "f16", "bf16", "fp8")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# dtype rounding (storage formats only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the storage array for ``dtype`` (bf16 as uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 upcast of a storage array."""
    if dtype == "bf16":
        return bf16_bits_to_f64(stored)
    return np.asarray(stored).astype(np.float64)


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to E4M3 codes (uint8), nearest-even, saturating
    at +-448 (the largest finite E4M3 value).  Normal codes are
    sign | (e + 7) << 3 | mantissa for |x| = (1 + mantissa / 8) * 2^e,
    e in [-6, 8]; below 2^-6 the codes are subnormal, |x| = mantissa * 2^-9."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), E4M3_MAX)
    # binade exponent of a (normal range), clamped to the subnormal binade
    _, ex = np.frexp(a)                       # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    steps = np.rint(a / np.ldexp(1.0, e - 3))  # multiples of the code spacing
    # steps in [8, 16] for normals (16: rounded up into the next binade),
    # [0, 8] in the subnormal binade (8: the smallest normal)
    up = steps >= 16
    e = np.where(up, e + 1, e)
    steps = np.where(up, 8, steps).astype(np.int64)
    normal = steps >= 8
    code = np.where(normal, ((e + 7) << 3) | (steps - 8), steps)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_e4m3(x32: np.ndarray) -> tuple[np.ndarray, float]:
    """Per-tensor FP8 storage: (codes, descale) with descale = amax / 448 as a
    float32 and codes = E4M3(x / descale); x ~= descale * decode(codes)."""
    amax = float(np.max(np.abs(x32))) if x32.size else 0.0
    descale = float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0
    return f32_to_e4m3(np.asarray(x32, dtype=np.float64) / descale), descale


def poison_value(dtype: str):
    if dtype == "bf16":
        return BF16_NAN
    if dtype == "fp8":
        return E4M3_NAN
    return np.nan


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Prefill:
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    n: int
    m: int
    d: int
    dv: int
    causal: bool
    seed: int
    hot: float = 1.0          # factor applied to Q and K
    ragged: tuple | None = None  # (lo, hi) inclusive bounds of left-padded lengths

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


@dataclasses.dataclass(frozen=True)
class Decode:
    name: str
    dtype: str
    num_seqs: int
    Hq: int
    Hkv: int
    d: int
    dv: int
    block_size: int
    len_lo: int
    len_hi: int
    max_blocks_per_seq: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five workloads (sizes as the benchmark spec gives them).
WORKLOADS = {
    "f32_256": Prefill("f32_256", "f32", 1, 1, 1, 256, 256, 64, 64, False, seed=1),
    "f32_256_hot": Prefill("f32_256_hot", "f32", 1, 1, 1, 256, 256, 64, 64, False, seed=1, hot=10.0),
    "bf16_b4_2048": Prefill("bf16_b4_2048", "bf16", 4, 32, 32, 2048, 2048, 128, 128, False, seed=2),
    "bf16_causal_8192": Prefill("bf16_causal_8192", "bf16", 1, 32, 32, 8192, 8192, 128, 128, True, seed=3),
    "bf16_ragged_b8_8192": Prefill("bf16_ragged_b8_8192", "bf16", 8, 32, 32, 8192, 8192, 128, 128, True,
                           seed=3, ragged=(1024, 8192)),
    "decode_64seq": Decode("decode_64seq", "bf16", 64, 32, 8, 128, 128, 16, 512, 8192, 512, seed=4),
    "f16_hot_causal_16384": Prefill("f16_hot_causal_16384", "f16", 1, 16, 16, 16384, 16384, 128, 128, True, seed=5, hot=10.0),
    # the bf16 2048-token prefill with FP8 (E4M3) storage
    "fp8_b4_2048": Prefill("fp8_b4_2048", "fp8", 4, 32, 32, 2048, 2048, 128, 128, False, seed=2),
}


def _normals(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def make_prefill(w: Prefill) -> dict:
    """Draw Q, K, V (and ragged lengths) for a prefill workload.

    Returns storage arrays ``q``, ``k``, ``v`` (bf16 as uint16 bits),
    ``seq_lens`` (int32 [B] or None) and ``pads`` (int [B] or None: the number
    of leading padding rows of each sequence, N - L_b).
    """
    rng = np.random.default_rng(w.seed)
    q32 = _normals(rng, (w.B, w.Hq, w.n, w.d))
    k32 = _normals(rng, (w.B, w.Hkv, w.m, w.d))
    v32 = _normals(rng, (w.B, w.Hkv, w.m, w.dv))
    if w.hot != 1.0:
        f = np.float32(w.hot)
        q32 *= f
        k32 *= f
    seq_lens = pads = None
    if w.ragged is not None:
        lo, hi = w.ragged
        seq_lens = rng.integers(lo, hi, size=w.B, endpoint=True).astype(np.int32)
        pads = (w.n - seq_lens).astype(np.int64)
    out = {"seq_lens": seq_lens, "pads": pads}
    if w.dtype == "fp8":
        # per-tensor scaling over the real (non-padding) entries
        for name, x32 in (("q", q32), ("k", k32), ("v", v32)):
            if pads is not None:
                for b, p in enumerate(pads):
                    x32[b, :, :p] = 0.0
            codes, descale = quantize_e4m3(x32)
            out[name], out[name + "_descale"] = codes, descale
    else:
        out["q"], out["k"], out["v"] = store(q32, w.dtype), store(k32, w.dtype), store(v32, w.dtype)
    del q32, k32, v32
    if pads is not None:
        pv = poison_value(w.dtype)
        for b, p in enumerate(pads):
            out["q"][b, :, :p] = pv
            out["k"][b, :, :p] = pv
            out["v"][b, :, :p] = pv
    return out


def make_prefill_custom(dtype, B, Hq, Hkv, n, m, d, dv, seed, hot=1.0, lens=None,
                        ragged=None) -> dict:
    """Same recipe at arbitrary (small) sizes, for parity tests."""
    w = Prefill("custom", dtype, B, Hq, Hkv, n, m, d, dv, False, seed, hot, ragged)
    out = make_prefill(w)
    if lens is not None:
        lens = np.asarray(lens, dtype=np.int32)
        out["seq_lens"] = lens
        out["pads"] = (n - lens).astype(np.int64)
        pv = poison_value(dtype)
        for b, p in enumerate(out["pads"]):
            out["q"][b, :, :p] = pv
            out["k"][b, :, :p] = pv
            out["v"][b, :, :p] = pv
    return out


def make_decode(w: Decode, seq_lens=None) -> dict:
    """Draw a paged GQA decode batch.

    Layout: q [S, Hq, d]; k_cache [NB, bs, Hkv, d]; v_cache [NB, bs, Hkv, dv];
    block_table int32 [S, max_blocks_per_seq] (physical block ids, -1 past the
    sequence's last block); seq_lens int32 [S].  Physical blocks are a seeded
    random permutation of 0..NB-1 dealt to the sequences in order.  Cache slots
    past a sequence's length are NaN.
    """
    rng = np.random.default_rng(w.seed)
    q32 = _normals(rng, (w.num_seqs, w.Hq, w.d))
    if seq_lens is None:
        seq_lens = rng.integers(w.len_lo, w.len_hi, size=w.num_seqs, endpoint=True)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    bs = w.block_size
    nblk = (seq_lens + bs - 1) // bs
    if nblk.max(initial=0) > w.max_blocks_per_seq:
        raise ValueError("sequence longer than max_blocks_per_seq * block_size")
    NB = int(nblk.sum())
    NBa = max(NB, 1)
    k32 = _normals(rng, (NBa, bs, w.Hkv, w.d))
    v32 = _normals(rng, (NBa, bs, w.Hkv, w.dv))
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((w.num_seqs, w.max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for s in range(w.num_seqs):
        c = int(nblk[s])
        table[s, :c] = perm[pos:pos + c]
        pos += c
    q, kc, vc = store(q32, w.dtype), store(k32, w.dtype), store(v32, w.dtype)
    del q32, k32, v32
    pv = poison_value(w.dtype)
    for s in range(w.num_seqs):
        c = int(nblk[s])
        tail = int(seq_lens[s]) - (c - 1) * bs if c else bs
        if c and tail < bs:
            last = table[s, c - 1]
            kc[last, tail:] = pv
            vc[last, tail:] = pv
    return {"q": q, "k_cache": kc, "v_cache": vc, "block_table": table,
            "seq_lens": seq_lens.astype(np.int32), "num_blocks": NBa}


def make_paged_chunk(w: Decode, n: int, seq_lens=None) -> dict:
    """make_decode's cache, block table and lengths, with a chunk of n query
    tokens per sequence, q [S, Hq, n, d], drawn from a second stream (seed + 1)
    in place of the single decode token."""
    x = make_decode(w, seq_lens)
    rng = np.random.default_rng(w.seed + 1)
    x["q"] = store(_normals(rng, (w.num_seqs, w.Hq, n, w.d)), w.dtype)
    return x


def paged_prefill_flops(seq_lens, n: int, Hq: int, d: int, dv: int, causal: bool = True) -> float:
    """(2d + 2dv) per (query, allowed key) pair of a chunk of n rows at the end
    of each sequence."""
    pairs = 0
    for L in np.asarray(seq_lens, dtype=np.int64):
        L = int(L)
        for i in range(max(0, n - L), n):
            pairs += (L - n + i + 1) if causal else L
    return float(pairs) * Hq * (2 * d + 2 * dv)


def prefill_flops(w: Prefill, seq_lens=None) -> float:
    """Algorithmic FLOPs: 2*d + 2*dv per unmasked (query, key) pair."""
    per_pair = 2 * w.d + 2 * w.dv
    if not w.causal:
        pairs = w.B * w.Hq * w.n * w.m
    elif seq_lens is None:
        pairs = w.B * w.Hq * w.n * (w.n + 1) // 2
    else:
        L = np.asarray(seq_lens, dtype=np.int64)
        pairs = int(w.Hq * np.sum(L * (L + 1) // 2))
    return float(per_pair) * float(pairs)


def decode_bytes(w: Decode, seq_lens) -> int:
    """Algorithmic HBM bytes of one decode call: the K/V rows read once, q, o,
    the block-table entries used and seq_lens."""
    L = np.asarray(seq_lens, dtype=np.int64)
    e = ELEM_BYTES[w.dtype]
    kv = int(L.sum()) * w.Hkv * (w.d + w.dv) * e
    qo = w.num_seqs * w.Hq * (w.d + w.dv) * e
    bt = int(((L + w.block_size - 1) // w.block_size).sum()) * 4
    return kv + qo + bt + 4 * w.num_seqs
