#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

One step = one prefill call (bf16, B=4, H=32, n=m=2048, d=128, non-causal, the
workload the headline metric is quoted on) followed by one paged GQA decode call
(64 sequences, 32 query / 8 KV heads, d=128, blocks of 16, lengths in
[512, 8192]).  Inputs are seeded synthetic tensors resident in device memory
before timing starts.  Prints one JSON line:

  value     prefill TFLOP/s (algorithmic: 4*d FLOP per (query, key) pair)
  roofline  the prefill kernel against the bf16 dense MFMA peak
  decode    paged decode GB/s (algorithmic bytes) against HBM peak
  cpu_baseline  the float64 oracle on a bounded sample, on this host's cores
After the timed steps, the same prefill is also timed as four key-range pieces
plus their merge, as a paged causal chunk over the decode cache, and with FP8
(E4M3) inputs against the FP8 MFMA peak; the causal prefill B=1 H=32
n=m=8192 is timed beside its dense twin, and the hot fp16 causal prefill
B=1 H=16 n=m=16384 with its count of non-finite outputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
PREFILL_SOURCES = ["tiled_online_softmax_04_amd/csrc/fa_prefill.hip",
                   "tiled_online_softmax_04_amd/csrc/fa_lds.h",
                   "tiled_online_softmax_04_amd/csrc/fa_common.h"]
FP8_SOURCES = ["tiled_online_softmax_04_amd/csrc/fa_prefill_fp8.hip",
               "tiled_online_softmax_04_amd/csrc/fa_lds.h",
               "tiled_online_softmax_04_amd/csrc/fa_common.h"]
DECODE_SOURCES = ["tiled_online_softmax_04_amd/csrc/fa_decode.hip",
                  "tiled_online_softmax_04_amd/csrc/fa_common.h"]


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, paths):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the summary is absent or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(paths):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, x, budget_s: float):
    """Time the float64 oracle on whole (batch, head) slices of the workload until
    about `budget_s` seconds of CPU work, and scale to TFLOP/s."""
    import oracle
    from tiled_online_softmax_04_amd import inputs as gen
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    heads = [(b, h) for b in range(w.B) for h in range(w.Hq)]
    done, t_used, flops = 0, 0.0, 0.0
    per_head = 4.0 * w.n * w.m * w.d
    for b, h in heads:
        q = gen.to_f64(x["q"][b:b + 1, h:h + 1], w.dtype)
        k = gen.to_f64(x["k"][b:b + 1, h:h + 1], w.dtype)
        v = gen.to_f64(x["v"][b:b + 1, h:h + 1], w.dtype)
        t0 = time.perf_counter()
        oracle.attention(q, k, v, w.scale, w.causal)
        t_used += time.perf_counter() - t0
        done += 1
        flops += per_head
        if t_used >= budget_s:
            break
    return {"value": flops / t_used / 1e12, "unit": "TFLOP/s",
            "cores": int(min(threads, len(os.sched_getaffinity(0)))), "kind": "oracle",
            "sample": f"{done} of {len(heads)} (batch, head) slices of the same workload, "
                      f"float64, {t_used:.1f} s"}


def time_key_split(fa, q, k, v, wp, iters: int):
    """The same prefill as four 512-key pieces (fa_fwd_partial) merged by
    fa_merge; timed outside the step, after it, with HIP events."""
    import torch
    if iters <= 0:
        return None
    bounds = [0, 512, 1024, 1536, 2048]
    B, Hq, n, dv = q.shape
    o_parts = torch.empty((4, B, Hq, n, dv), dtype=torch.float32, device=q.device)
    l_parts = torch.empty((4, B, Hq, n), dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)

    def run(ev=None):
        if ev is not None:
            ev[0].record()
        for i, (lo, hi) in enumerate(zip(bounds[:-1], bounds[1:])):
            fa.fwd_partial(q, k, v, lo, hi, scale=wp.scale, out=o_parts[i], lse=l_parts[i])
        if ev is not None:
            ev[1].record()
        fa.merge(o_parts, l_parts, out=out)
        if ev is not None:
            ev[2].record()

    for _ in range(max(10, iters // 2)):
        run()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    part_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    merge_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    rows = B * Hq * n
    merge_bytes = 4 * rows * (dv + 1) * 4 + rows * dv * 2
    from tiled_online_softmax_04_amd import inputs as gen
    flops = gen.prefill_flops(wp)
    return {"workload": "the prefill above as keys [0,512) [512,1024) [1024,1536) [1536,2048) "
                        "through fa_fwd_partial, then fa_merge",
            "tflops_total": round(flops / ((part_ms + merge_ms) * 1e-3) / 1e12, 2),
            "tflops_pieces": round(flops / (part_ms * 1e-3) / 1e12, 2),
            "pieces_ms": round(part_ms, 5), "merge_ms": round(merge_ms, 5),
            "merge_gbps": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1),
            "merge_bytes": merge_bytes, "iters": iters}


def time_paged_prefill(fa, wd, kc, vc, bt, sl, seq_lens, iters: int, n: int = 512):
    """A 512-token causal chunk per sequence over the decode workload's paged
    cache (the chunk being the last 512 tokens of each sequence); HIP events
    around fa_paged_prefill, after the step."""
    import torch
    from tiled_online_softmax_04_amd import inputs as gen
    if iters <= 0:
        return None
    g = torch.Generator(device="cpu").manual_seed(wd.seed + 1)
    q = torch.randn((wd.num_seqs, wd.Hq, n, wd.d), generator=g).to(torch.bfloat16).to(kc.device)
    out = torch.empty((wd.num_seqs, wd.Hq, n, wd.dv), dtype=q.dtype, device=q.device)
    for _ in range(max(10, iters // 2)):
        fa.paged_prefill(q, kc, vc, bt, sl, wd.block_size, scale=wd.scale, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fa.paged_prefill(q, kc, vc, bt, sl, wd.block_size, scale=wd.scale, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    flops = gen.paged_prefill_flops(seq_lens, n, wd.Hq, wd.d, wd.dv, causal=True)
    return {"workload": f"paged prefill bf16: a {n}-token causal chunk at the end of each of the "
                        "decode workload's 64 sequences (Hq=32, Hkv=8, d=128, 16-token blocks, "
                        "random placement)",
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "ms": round(ms, 5), "flop": flops,
            "iters": iters}


def time_fp8(fa, iters: int):
    """The headline prefill with Q, K, V stored as FP8 E4M3 (per-tensor
    descales) and a bf16 output; HIP events around each fa_fwd_fp8 call."""
    import torch
    from tiled_online_softmax_04_amd import inputs as gen
    if iters <= 0:
        return None
    w = gen.WORKLOADS["cfg2_fp8"]
    x = gen.make_prefill(w)
    q8, k8, v8 = (torch.from_numpy(x[t]).cuda() for t in ("q", "k", "v"))
    out = torch.empty((w.B, w.Hq, w.n, w.dv), dtype=torch.bfloat16, device=q8.device)

    def run():
        fa.fwd_fp8(q8, k8, v8, x["q_descale"], x["k_descale"], x["v_descale"], scale=w.scale,
                   out=out)

    for _ in range(max(200, iters)):   # steady clocks after the other legs
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record()
        run()
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    tflops = gen.prefill_flops(w) / (ms * 1e-3) / 1e12
    return {"workload": "the prefill above (B=4 H=32 n=m=2048 d=dv=128 non-causal) with Q, K, V "
                        "stored as FP8 E4M3 with per-tensor descales, bf16 output",
            "tflops": round(tflops, 2), "ms": round(ms, 5), "iters": iters,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                         "traffic": read_traffic("fa_fwd_fp8_cfg2_traffic.txt", FP8_SOURCES),
                         "kernel": "fa_fwd_fp8<128,false,false,2> (non-causal, no padding, "
                                   "bf16 out)"}}


def time_causal(fa, iters: int):
    """The causal bf16 prefill B=1 H=32 n=m=8192 d=128, and the same inputs
    without the mask (its dense twin); HIP events around each fa_fwd call.
    The causal FLOPs count only unmasked pairs."""
    import torch
    from tiled_online_softmax_04_amd import inputs as gen
    if iters <= 0:
        return None
    w = gen.WORKLOADS["cfg3"]
    x = gen.make_prefill(w)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x[t]).view(np.int16)).cuda()
               .view(torch.bfloat16) for t in ("q", "k", "v"))
    out = torch.empty_like(q)
    res = {}
    for causal in (True, False):
        for _ in range(max(50, iters)):
            fa.fwd(q, k, v, scale=w.scale, causal=causal, out=out)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(iters)]
        for e0, e1 in evs:
            e0.record()
            fa.fwd(q, k, v, scale=w.scale, causal=causal, out=out)
            e1.record()
        torch.cuda.synchronize()
        res[causal] = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    flop_causal = gen.prefill_flops(w)
    flop_dense = 4.0 * w.B * w.Hq * w.n * w.m * w.d
    del q, k, v, out
    # the hot long-context case: fp16, Q and K x10 (scores far past the fp16
    # exp overflow point); the whole output must be finite
    w5 = gen.WORKLOADS["cfg5"]
    x5 = gen.make_prefill(w5)
    q5, k5, v5 = (torch.from_numpy(np.ascontiguousarray(x5[t])).cuda() for t in ("q", "k", "v"))
    out5 = torch.empty_like(q5)
    for _ in range(max(20, iters)):
        fa.fwd(q5, k5, v5, scale=w5.scale, causal=True, out=out5)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(iters)]
    for e0, e1 in evs:
        e0.record()
        fa.fwd(q5, k5, v5, scale=w5.scale, causal=True, out=out5)
        e1.record()
    torch.cuda.synchronize()
    ms5 = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    nonfinite5 = int((~torch.isfinite(out5)).sum().item())
    return {"workload": "causal prefill bf16 B=1 H=32 n=m=8192 d=dv=128, and its dense twin "
                        "(the same inputs without the mask)",
            "tflops": round(flop_causal / (res[True] * 1e-3) / 1e12, 2),
            "ms": round(res[True], 5),
            "dense_twin_tflops": round(flop_dense / (res[False] * 1e-3) / 1e12, 2),
            "dense_twin_ms": round(res[False], 5),
            "time_ratio": round(res[True] / res[False], 4), "iters": iters,
            "hot_fp16_16384": {"workload": "causal prefill fp16 B=1 H=16 n=m=16384 d=dv=128, Q and "
                                           "K drawn x10 (scores up to ~300)",
                               "tflops": round(gen.prefill_flops(w5) / (ms5 * 1e-3) / 1e12, 2),
                               "ms": round(ms5, 5), "nonfinite_outputs": nonfinite5}}


def peak_memory(fa, sizes=(512, 2048, 8192), d=128):
    """Peak device memory of one attention head, beyond its inputs and output:
    the tiled library call against the plain three-step evaluation that keeps
    S and P (float32) in device memory (exercise 3 of the S12 chapter)."""
    import torch
    dev = torch.device("cuda:0")
    out = []
    for n in sizes:
        g = torch.Generator(device="cpu").manual_seed(n)
        q, k, v = (torch.randn((1, 1, n, d), generator=g).to(torch.bfloat16).to(dev)
                   for _ in range(3))
        o = torch.empty_like(q)
        scale = 1.0 / math.sqrt(d)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        fa.fwd(q, k, v, scale=scale, out=o)
        torch.cuda.synchronize()
        flash_extra = torch.cuda.max_memory_allocated(dev) - base
        kt = k.float()[0, 0].t().contiguous()

        def naive():
            s = (q.float()[0, 0] @ kt) * scale      # S [n, n] float32
            p_ = torch.softmax(s, dim=-1)           # P [n, n] float32
            return (p_ @ v.float()[0, 0]).to(torch.bfloat16)

        naive()  # first use sets up the matrix library's own workspace
        torch.cuda.synchronize()
        base2 = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        o2 = naive()
        torch.cuda.synchronize()
        naive_extra = torch.cuda.max_memory_allocated(dev) - base2
        out.append({"n": n, "flash_extra_bytes": int(flash_extra),
                    "naive_extra_bytes": int(naive_extra),
                    "n2_float32_bytes": 4 * n * n})
        del o2, kt, q, k, v, o
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU needs a few hundred calls to "
                         "reach steady clocks")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 skips it)")
    ap.add_argument("--key-split-iters", type=int, default=30,
                    help="timed runs of the key-split, paged-prefill and FP8 variants after the "
                         "step (0 skips them)")
    ap.add_argument("--causal-iters", type=int, default=20,
                    help="timed runs of the causal 8192 prefill and its dense twin after the "
                         "step (0 skips them)")
    ap.add_argument("--peak-memory", type=int, default=1,
                    help="1: also report peak device memory, tiled vs naive, at n = 512, 2048, "
                         "8192 (0 skips it)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one device copy of this size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures a single GPU; runs on more than one GPU are not part of "
              "this build (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_online_softmax_04_amd import fa
    from tiled_online_softmax_04_amd import inputs as gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(a, dtype):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    wp = gen.WORKLOADS["cfg2"]
    xp = gen.make_prefill(wp)
    q, k, v = (to_dev(xp[n], wp.dtype) for n in ("q", "k", "v"))
    o = torch.empty_like(q)

    wd = gen.WORKLOADS["cfg4"]
    xd = gen.make_decode(wd)
    dq = to_dev(xd["q"], wd.dtype)
    kc, vc = to_dev(xd["k_cache"], wd.dtype), to_dev(xd["v_cache"], wd.dtype)
    bt = torch.from_numpy(xd["block_table"]).to(dev)
    sl = torch.from_numpy(xd["seq_lens"]).to(dev)
    do = torch.empty((wd.num_seqs, wd.Hq, wd.dv), dtype=dq.dtype, device=dev)
    ws_bytes = fa.paged_decode_workspace_size(wd.num_seqs, wd.Hq, wd.Hkv, wd.dv,
                                              wd.max_blocks_per_seq, wd.block_size)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.fwd(q, k, v, scale=wp.scale, causal=wp.causal, out=o)
        if ev is not None:
            ev[1].record()
        fa.paged_decode(dq, kc, vc, bt, sl, wd.block_size, scale=wd.scale, out=do, workspace=ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    pre_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    flops = gen.prefill_flops(wp)
    dbytes = gen.decode_bytes(wd, xd["seq_lens"])
    pre_tflops = flops / (pre_ms.mean() * 1e-3) / 1e12
    dec_gbps = dbytes / (dec_ms.mean() * 1e-3) / 1e9

    key_split = time_key_split(fa, q, k, v, wp, args.key_split_iters)
    paged = time_paged_prefill(fa, wd, kc, vc, bt, sl, xd["seq_lens"], args.key_split_iters)
    fp8 = time_fp8(fa, args.key_split_iters)
    causal = time_causal(fa, args.causal_iters)
    mem = peak_memory(fa) if args.peak_memory else None

    traffic = read_traffic("fa_fwd_mfma_bf16_cfg2_traffic.txt", PREFILL_SOURCES)
    dec_traffic = read_traffic("fa_decode_cfg4_traffic.txt", DECODE_SOURCES)

    baseline = None
    if args.cpu_budget > 0:
        baseline = cpu_baseline(wp, xp, args.cpu_budget)

    out = {
        "metric": "attn fwd TFLOP/s + % bf16 MFMA peak; paged decode GB/s + % HBM peak",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill bf16 B=4 H=32 n=m=2048 d=dv=128 non-causal, "
                               "then paged GQA decode bf16 64 seqs Hq=32 Hkv=8 d=128 block 16 "
                               "lengths U[512,8192]",
                   "prefill_flop": flops, "decode_bytes": dbytes, "seed_prefill": wp.seed,
                   "seed_decode": wd.seed},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "fa_fwd_mfma<BF16,128,false,false,false,false> (non-causal, no padding, full key range, contiguous)",
                     "avg_launch_ms": round(float(pre_ms.mean()), 5)},
        "decode": {"value": round(dec_gbps, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 1),
                                "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(dec_gbps / PEAK_HBM_GBPS, 4),
                                "traffic": dec_traffic,
                                "kernels": "fa_decode_split + fa_decode_merge",
                                "avg_call_ms": round(float(dec_ms.mean()), 5)}},
        "cpu_baseline": baseline,
        "key_split": key_split,
        "paged_prefill": paged,
        "fp8": fp8,
        "causal": causal,
        "peak_memory": mem,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
