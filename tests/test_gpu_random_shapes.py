"""GPU parity on seeded random shapes: fa_fwd against the float64 oracle on
every output element, over a spread of batch and head counts (grouped-query
included), query and key lengths with ragged tails, head dims, 16-bit types,
causal masks and left-padded batches.  The last cases have enough query tiles
(512 and more) that the dense non-causal calls take the persistent form."""
import numpy as np
import pytest

import oracle
from tiled_online_softmax_04_amd import fa
from tiled_online_softmax_04_amd import inputs as gen

from gpu_util import assert_parity, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(28):
        dtype = ["bf16", "f16"][int(rng.integers(2))]
        d = [64, 128][int(rng.integers(2))]
        B = int(rng.integers(1, 4))
        Hkv = [1, 2, 4][int(rng.integers(3))]
        Hq = Hkv * [1, 2, 4, 8][int(rng.integers(4))]
        causal = bool(rng.integers(2))
        n = int(rng.integers(1, 1100))
        ragged = rng.random() < 0.3
        m = n if (causal or ragged) else int(rng.integers(1, 1100))
        lens = [int(x) for x in rng.integers(0, n + 1, size=B)] if ragged else None
        out.append((f"r{i:02d}_{dtype}_d{d}_B{B}_H{Hq}x{Hkv}_n{n}_m{m}"
                    f"{'_causal' if causal else ''}{'_pad' if ragged else ''}",
                    dtype, B, Hq, Hkv, n, m, d, causal, lens, int(rng.integers(1 << 30))))
    # enough units (B * Hq * ceil(n / 256) >= 512) for the persistent dense form
    for i, (dtype, d, B, Hq, Hkv, n, m) in enumerate([("bf16", 128, 2, 64, 8, 1100, 900),
                                                     ("f16", 64, 1, 128, 32, 1030, 1030),
                                                     ("bf16", 64, 3, 48, 48, 900, 1),
                                                     ("f16", 128, 2, 80, 16, 800, 513)]):
        out.append((f"p{i}_{dtype}_d{d}_B{B}_H{Hq}x{Hkv}_n{n}_m{m}", dtype, B, Hq, Hkv, n, m, d,
                    False, None, 1000 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_shape(case):
    import torch
    name, dtype, B, Hq, Hkv, n, m, d, causal, lens, seed = case
    say(f"[random] {name}")
    x = gen.make_prefill_custom(dtype, B, Hq, Hkv, n, m, d, d, seed=seed % 100000, lens=lens)
    scale = float(np.float32(1 / np.sqrt(d)))
    q, k, v = (to_dev(x[t], dtype) for t in ("q", "k", "v"))
    sl = None if x["seq_lens"] is None else torch.from_numpy(x["seq_lens"]).cuda()
    o = fa.fwd(q, k, v, scale=scale, causal=causal, seq_lens=sl)
    torch.cuda.synchronize()
    got = to_f64(o, dtype)
    qf, kf, vf = (gen.to_f64(x[t], dtype) for t in ("q", "k", "v"))
    ref = oracle.attention(qf, kf, vf, scale, causal, pads=x["pads"])
    assert_parity(got, ref, dtype, name)
    if x["pads"] is not None:
        for b, p in enumerate(x["pads"]):
            assert np.all(got[b, :, :p] == 0), "padding rows must be exactly 0"
