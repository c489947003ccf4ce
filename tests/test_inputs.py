"""Seeded input generators: determinism, storage rounding, poison placement."""
import math

import numpy as np
import pytest
import torch

from tiled_online_softmax_04_amd import inputs as gen


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-30, -3.3895e38], np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = gen.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_f16_rounding_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(100000).astype(np.float32) * 30
    ours = gen.store(x, "f16")
    theirs = torch.from_numpy(x).to(torch.float16).numpy()
    assert np.array_equal(ours.view(np.uint16), theirs.view(np.uint16))


def test_prefill_deterministic_and_shaped():
    w = gen.Prefill("t", "bf16", 2, 4, 2, 40, 40, 64, 64, True, seed=9, hot=10.0, ragged=(5, 40))
    a, b = gen.make_prefill(w), gen.make_prefill(w)
    for key in ("q", "k", "v", "seq_lens"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (2, 4, 40, 64) and a["k"].shape == (2, 2, 40, 64)
    assert a["q"].dtype == np.uint16
    assert np.all((a["seq_lens"] >= 5) & (a["seq_lens"] <= 40))
    for bi, p in enumerate(a["pads"]):
        assert np.all(a["k"][bi, :, :p] == gen.BF16_NAN)
        if p < 40:
            assert np.isfinite(gen.to_f64(a["k"][bi, :, p:], "bf16")).all()
    # hot: Q, K scaled by 10, V not
    q = gen.to_f64(a["q"][0, :, a["pads"][0]:], "bf16")
    v = gen.to_f64(a["v"][0, :, a["pads"][0]:], "bf16")
    assert q.std() > 5 and v.std() < 2


def test_scale_is_float32_rounded():
    """A float64 1/sqrt(d) silently promotes fp32 arithmetic (10100.com section
    4); the workloads carry the float32 value the kernel receives."""
    w = gen.WORKLOADS["bf16_b4_2048"]
    assert w.scale == float(np.float32(1 / math.sqrt(128)))


def test_decode_table_is_a_permutation_with_poisoned_tails():
    w = gen.Decode("t", "bf16", 5, 8, 2, 64, 64, 16, 1, 70, 5, seed=3)
    x = gen.make_decode(w)
    L = x["seq_lens"].astype(int)
    nblk = (L + 15) // 16
    used = np.concatenate([x["block_table"][s, :nblk[s]] for s in range(5)])
    assert sorted(used.tolist()) == list(range(int(nblk.sum())))
    for s in range(5):
        assert np.all(x["block_table"][s, nblk[s]:] == -1)
        tail = L[s] - (nblk[s] - 1) * 16
        last = x["block_table"][s, nblk[s] - 1]
        if tail < 16:
            assert np.all(x["k_cache"][last, tail:] == gen.BF16_NAN)
        assert np.isfinite(gen.to_f64(x["k_cache"][last, :tail], "bf16")).all()


def test_algorithmic_counts():
    assert gen.prefill_flops(gen.WORKLOADS["bf16_b4_2048"]) == 4 * 4 * 32 * 2048 * 2048 * 128
    assert abs(gen.prefill_flops(gen.WORKLOADS["bf16_b4_2048"]) - 2.749e11) < 1e9
    assert abs(gen.prefill_flops(gen.WORKLOADS["bf16_causal_8192"]) - 5.498e11) < 1e9
    assert abs(gen.prefill_flops(gen.WORKLOADS["f16_hot_causal_16384"]) - 1.0996e12) < 1e9
    w = gen.WORKLOADS["decode_64seq"]
    L = np.full(64, 16 * 10)
    assert gen.decode_bytes(w, L) == (64 * 160 * 8 * 256 * 2 + 64 * 32 * 256 * 2
                                      + 64 * 10 * 4 + 64 * 4)


@pytest.mark.parametrize("name", ["f32_256", "f32_256_hot"])
def test_small_workload_values(name):
    w = gen.WORKLOADS[name]
    x = gen.make_prefill(w)
    assert x["q"].dtype == np.float32 and x["q"].shape == (1, 1, 256, 64)
    s = x["q"][0, 0].astype(np.float64) @ x["k"][0, 0].astype(np.float64).T * w.scale
    if w.hot > 1:
        assert np.abs(s).max() > 200      # 'hot' scores of a few hundred
    else:
        assert np.abs(s).max() < 10


def test_paged_chunk_shares_the_decode_cache():
    w = gen.Decode("t", "bf16", 3, 4, 2, 64, 64, 16, 10, 90, 8, seed=11)
    a = gen.make_paged_chunk(w, 5)
    b = gen.make_paged_chunk(w, 5)
    d = gen.make_decode(w)
    assert a["q"].shape == (3, 4, 5, 64)
    assert np.array_equal(a["q"], b["q"])
    for k in ("k_cache", "v_cache", "block_table", "seq_lens"):
        assert np.array_equal(a[k], d[k], equal_nan=True) if a[k].dtype.kind == "f" else \
            np.array_equal(a[k], d[k])


def test_paged_prefill_flops_closed_form():
    # causal: row i of a chunk of n at the end of L tokens sees L - n + i + 1 keys
    L, n = 100, 30
    pairs = sum(L - n + i + 1 for i in range(n))
    assert gen.paged_prefill_flops([L], n, 2, 64, 64) == pairs * 2 * (4 * 64)
    assert gen.paged_prefill_flops([L], n, 1, 64, 64, causal=False) == n * L * 4 * 64
    assert gen.paged_prefill_flops([3], 5, 1, 1, 1) == (1 + 2 + 3) * 4  # rows before 0 skipped


def test_e4m3_rounding_matches_torch_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s
                        for s in (0.003, 0.3, 30.0, 150.0)])
    x = np.clip(x, -448, 448)
    ours = gen.f32_to_e4m3(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_ties_and_saturation():
    # halfway cases go to the even mantissa; beyond 448 saturates
    x = np.array([1.0625, 1.1875, 272.0, 2.0 ** -10, 3 * 2.0 ** -10, 464.0, 1000.0, -1e9,
                  0.0, -0.0], np.float32)
    want = [0x38, 0x3A, 0x78, 0x00, 0x02, 0x7E, 0x7E, 0xFE, 0x00, 0x80]
    assert gen.f32_to_e4m3(x).tolist() == want


def test_fp8_prefill_per_tensor_scaling_and_poison():
    w = gen.Prefill("t", "fp8", 2, 4, 2, 40, 40, 64, 64, True, seed=9, ragged=(5, 40))
    a, b = gen.make_prefill(w), gen.make_prefill(w)
    for key in ("q", "k", "v", "seq_lens"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].dtype == np.uint8 and a["k"].shape == (2, 2, 40, 64)
    for name in ("q", "k", "v"):
        d = a[name + "_descale"]
        assert d == float(np.float32(d)) and d > 0
        codes = a[name]
        live = np.concatenate([codes[bi, :, p:].ravel() for bi, p in enumerate(a["pads"])])
        # the largest real magnitude maps to (about) the top code, 448
        assert (live & 0x7F).max() in (0x7E, 0x7D)
        for bi, p in enumerate(a["pads"]):
            assert np.all(codes[bi, :, :p] == gen.E4M3_NAN)
