"""GPU parity of the paged chunked prefill (fa_paged_prefill): a chunk of n
query tokens at the end of each sequence over a block-table KV cache, against
the float64 oracle's paged_prefill on the same seeded inputs (block tables are
random permutations; cache tails and unused table entries are poisoned).  Bar:
max abs <= 1e-2 and mean abs <= 1e-3 for bf16 / fp16, no inf/NaN, rows with no
keys exactly 0."""
import dataclasses

import numpy as np
import pytest

import oracle
from tiled_online_softmax_04_amd import fa
from tiled_online_softmax_04_amd import inputs as gen

from gpu_util import assert_parity, assert_whole, error_sums, pooled, say, to_dev, to_f64

pytestmark = pytest.mark.gpu


def run(x, dtype, bs, scale, causal):
    import torch
    q = to_dev(x["q"], dtype)
    kc, vc = to_dev(x["k_cache"], dtype), to_dev(x["v_cache"], dtype)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seq_lens"]).cuda()
    o = fa.paged_prefill(q, kc, vc, bt, sl, bs, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o


def oracle_of(x, dtype, bs, scale, causal):
    return oracle.paged_prefill(gen.to_f64(x["q"], dtype), gen.to_f64(x["k_cache"], dtype),
                                gen.to_f64(x["v_cache"], dtype), x["block_table"], x["seq_lens"],
                                bs, scale, causal)


CASES = [
    # name, dtype, S, Hq, Hkv, d, bs, lens, maxb, n, causal
    ("bf16_bs16_causal", "bf16", 3, 8, 2, 128, 16, [300, 77, 700], 48, 77, True),
    ("bf16_bs16_short_seq", "bf16", 2, 4, 4, 128, 16, [40, 400], 32, 100, True),   # n > L
    ("f16_bs7_causal", "f16", 3, 4, 1, 128, 7, [130, 7, 301], 50, 64, True),
    ("bf16_bs32_noncausal", "bf16", 2, 8, 8, 64, 32, [257, 64], 16, 90, False),
    ("f16_d64_gqa_causal", "f16", 4, 16, 4, 64, 16, [1, 33, 129, 250], 20, 17, True),
    ("bf16_whole_sequence", "bf16", 2, 2, 2, 128, 16, [256, 256], 16, 256, True),
    # block sizes around the 64-key tile: a block per tile, blocks wider than a
    # tile, one key per block, and a ragged last tile in each
    ("bf16_bs64_causal", "bf16", 2, 4, 2, 128, 64, [450, 130], 8, 200, True),
    ("f16_bs128_noncausal", "f16", 2, 4, 4, 128, 128, [333, 129], 4, 70, False),
    ("bf16_bs1_causal", "bf16", 2, 2, 1, 64, 1, [150, 70], 160, 40, True),
    # block tables of up to 8192 entries take the pipelined loop (the table fills the
    # LDS beside the four-stage ring at 8192); larger ones the one-tile-per-barrier loop
    ("bf16_table_8192", "bf16", 2, 4, 1, 128, 16, [500, 1200], 8192, 150, True),
    ("bf16_table_9000", "bf16", 2, 4, 2, 128, 16, [900, 333], 9000, 200, True),
    ("f16_d64_table_12000_noncausal", "f16", 2, 8, 8, 64, 8, [1000, 50], 12000, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_prefill_small(case):
    name, dtype, S, Hq, Hkv, d, bs, lens, maxb, n, causal = case
    say(f"[paged prefill] {name}")
    w = gen.Decode(name, dtype, S, Hq, Hkv, d, d, bs, 1, 1, maxb, seed=sum(map(ord, name)))
    x = gen.make_paged_chunk(w, n, seq_lens=lens)
    scale = float(np.float32(1 / np.sqrt(d)))
    got = to_f64(run(x, dtype, bs, scale, causal), dtype)
    ref = oracle_of(x, dtype, bs, scale, causal)
    assert_parity(got, ref, dtype, name)
    for s, L in enumerate(lens):
        if n > L:
            assert np.all(got[s, :, :n - L] == 0), "rows before the sequence must be 0"


def _random_cases():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(16):
        dtype = ["bf16", "f16"][int(rng.integers(2))]
        d = [64, 128][int(rng.integers(2))]
        S = int(rng.integers(1, 5))
        Hkv = [1, 2, 4][int(rng.integers(3))]
        Hq = Hkv * [1, 2, 4][int(rng.integers(3))]
        bs = [1, 2, 8, 16, 32, 64, 128, 5, 12, 48][int(rng.integers(10))]
        lens = [int(x) for x in rng.integers(0, 900, size=S)]
        maxb = max(1, (max(lens) + bs - 1) // bs + int(rng.integers(0, 3)))
        n = int(rng.integers(1, 300))
        causal = bool(rng.integers(2))
        out.append((f"r{i:02d}_{dtype}_d{d}_S{S}_H{Hq}x{Hkv}_bs{bs}_n{n}{'_causal' if causal else ''}",
                    dtype, S, Hq, Hkv, d, bs, lens, maxb, n, causal))
    return out


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_paged_prefill_random(case):
    """Seeded random shapes (block sizes powers of two and not, empty and
    short sequences, chunks longer than their sequence): every output element
    against the oracle, rows before a sequence's first token exactly 0."""
    test_paged_prefill_small(case)


def test_chunk_of_one_is_the_decode():
    import torch
    w = gen.WORKLOADS["decode_64seq"]
    w = dataclasses.replace(w, num_seqs=8, len_lo=100, len_hi=3000, max_blocks_per_seq=200)
    x = gen.make_paged_chunk(w, 1)
    q = to_dev(x["q"], w.dtype)
    kc, vc = to_dev(x["k_cache"], w.dtype), to_dev(x["v_cache"], w.dtype)
    bt = torch.from_numpy(x["block_table"]).cuda()
    sl = torch.from_numpy(x["seq_lens"]).cuda()
    pre = fa.paged_prefill(q, kc, vc, bt, sl, w.block_size, scale=w.scale)[:, :, 0]
    dec = fa.paged_decode(q[:, :, 0].contiguous(), kc, vc, bt, sl, w.block_size, scale=w.scale)
    torch.cuda.synchronize()
    assert_parity(to_f64(pre, w.dtype), to_f64(dec, w.dtype), w.dtype, "n=1 prefill vs decode")


def test_full_size_chunk_whole_output():
    """The decode workload's cache (64 sequences, lengths in [512, 8192], 16-token
    blocks, random placement) with a 512-token causal chunk per sequence, in
    the launch the benchmark times: every output element against the oracle,
    one (sequence, KV head) at a time through the block table."""
    import torch
    w = gen.WORKLOADS["decode_64seq"]
    n = 512
    say("[paged prefill] decode_64seq cache, 512-token chunks")
    x = gen.make_paged_chunk(w, n)
    o = run(x, w.dtype, w.block_size, w.scale, True)
    got_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    del o
    group = w.Hq // w.Hkv

    def one(sg):
        s, g = sg
        L = int(x["seq_lens"][s])
        kk = gen.to_f64(oracle.gather_paged(x["k_cache"], x["block_table"][s], L, w.block_size,
                                            g), w.dtype)
        vv = gen.to_f64(oracle.gather_paged(x["v_cache"], x["block_table"][s], L, w.block_size,
                                            g), w.dtype)
        pos = np.arange(L - n, L)
        parts = []
        for h in range(g * group, (g + 1) * group):
            ref = oracle.attend(gen.to_f64(x["q"][s, h], w.dtype), pos, kk, vv, w.scale, True)
            parts.append(error_sums(gen.bf16_bits_to_f64(got_bits[s, h]), ref))
        return parts

    res = pooled(one, [(s, g) for s in range(w.num_seqs) for g in range(w.Hkv)])
    assert_whole([p for r in res for p in r], w.dtype, "decode_64seq cache, 512-token chunks")
