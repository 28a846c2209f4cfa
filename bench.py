#!/usr/bin/env python3
"""Benchmark of the paged GQA hot path on one MI355X.

A step is one pass of the decode path (decode kernel + split combine) over the
paged-decode workload: B=64 sequences, Hq=32, Hkv=8, D=128, page 16, context
lengths uniform in [512, 4096], bf16, pages scattered by a seeded
permutation. Inputs are resident in HBM before the timed region. ``value`` is
algorithmic KV bytes (every live K and V row read once) per second of
wall-clock step time. The same run also times causal prefill (B=4, S=2048,
Hq=32, Hkv=8, D=128, bf16, KV append included) and reports TFLOP/s for the
causal half of the attention flops, plus the float64 oracle on the host cores
as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--splits NS]
                       [--no-prefill] [--no-cpu-baseline] [--sweep]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import torch

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "decode KV GB/s (% HBM peak); prefill TFLOPS (% bf16 MFMA peak)"
DEFAULT_SPLITS = 4


def kv_bytes(x) -> int:
    """Algorithmic bytes of one decode pass: every live K and V row once."""
    T = int(x.context_lens.sum())
    hkv, d = x.k_cache.shape[1], x.k_cache.shape[3]
    return 2 * T * hkv * d * x.k_cache.element_size()


def prefill_flops(B, S, hq, d) -> float:
    """QK^T and PV flops of the causal half: 4*D*S(S+1)/2 per (b, head)."""
    return 4.0 * d * S * (S + 1) / 2 * B * hq


def event_times(fn, n, stream, flush=None):
    """Per-call durations (ms) from HIP events recorded on ``stream``."""
    ts = []
    for _ in range(n):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return ts


def cpu_baseline_decode(x_cpu, budget_s=12.0):
    import oracle  # test infrastructure: the float64 CPU oracle, timed as a baseline only
    B = x_cpu.q.shape[0]
    per_b = []
    t0w, t0c = time.perf_counter(), time.process_time()
    done_bytes = 0
    b = 0
    while time.perf_counter() - t0w < budget_s and b < B:
        T = int(x_cpu.context_lens[b])
        oracle.decode_paged(x_cpu.q[b:b + 1], x_cpu.k_cache, x_cpu.v_cache,
                            x_cpu.page_table[b:b + 1], x_cpu.context_lens[b:b + 1], x_cpu.scale)
        done_bytes += 2 * T * x_cpu.k_cache.shape[1] * x_cpu.k_cache.shape[3] * 2
        b += 1
    wall = time.perf_counter() - t0w
    cpu = time.process_time() - t0c
    return dict(value=done_bytes / wall / 1e9, unit="GB/s", cores=max(1, round(cpu / wall)),
                kind="oracle",
                sample=f"float64 oracle over the first {b} of {B} sequences of the decode "
                       f"workload ({done_bytes / 1e6:.1f} MB of KV) in {wall:.1f} s",
                host_cores=len(os.sched_getaffinity(0)))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=DEFAULT_SPLITS)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="extra lines for the split/batch sweeps")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(decode and prefill shard by sequence or KV head with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    import gqa_paged_kv_amd as g
    import synth
    g.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- decode workload (inputs resident in HBM) ----------------
    x = synth.config2(device=dev)
    ns = args.splits
    out = torch.empty_like(x.q)
    ws = g.alloc_workspace(x.q.shape[0], x.q.shape[1], x.q.shape[2], ns, dev) if ns > 1 else None
    nbytes = kv_bytes(x)

    def step():
        g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, num_splits=ns,
                       scale=x.scale, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ev_avg = statistics.fmean(ev)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (ev_avg * 1e-3) / 1e9

    # same launch preceded by a 512 MiB write that evicts L2 and the Infinity Cache
    scratch = torch.empty(512 * 2**20 // 4, dtype=torch.float32, device=dev)
    flushed = event_times(step, 30, stream, flush=lambda: scratch.zero_())
    flushed_med = statistics.median(flushed)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "paged GQA decode, B=64, Hq=32, Hkv=8, D=128, page 16, "
                        "T~U[512,4096], bf16, permuted pages",
            "num_splits": ns,
            "kv_bytes_per_step": nbytes,
            "total_context_tokens": int(x.context_lens.sum()),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "decode_paged_kernel<bf16,128,4> + combine_kernel (one decode call)",
            "event_avg_us": round(ev_avg * 1e3, 2),
        },
        "decode_flushed": {
            "median_us": round(flushed_med * 1e3, 2),
            "gbs": round(nbytes / (flushed_med * 1e-3) / 1e9, 1),
            "frac": round(nbytes / (flushed_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "each launch preceded by a 512 MiB write (L2 + Infinity Cache evicted)",
        },
    }
    del scratch

    # ---------------- prefill workload ----------------
    if not args.no_prefill:
        p = synth.config3(device=dev)
        pout = torch.empty_like(p.q)

        def pstep():
            g.prefill_causal(p.q, p.k, p.v, p.k_cache, p.v_cache, p.page_table, scale=p.scale,
                             out=pout)

        for _ in range(5):
            pstep()
        torch.cuda.synchronize()
        pt = event_times(pstep, 30, stream)
        pmed = statistics.median(pt)
        B, S, hq, d = p.q.shape
        fl = prefill_flops(B, S, hq, d)
        tf = fl / (pmed * 1e-3) / 1e12
        line["prefill"] = {
            "workload": "causal GQA prefill, B=4, S=2048, Hq=32, Hkv=8, D=128, bf16, "
                        "append to page-16 cache",
            "median_us": round(pmed * 1e3, 2),
            "tflops": round(tf, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": None,
                         "kernel": "append_kernel x2 + prefill_causal_kernel<4> (one call)"},
            "flops_per_call": fl,
        }
        del p, pout

    # ---------------- CPU baseline: the float64 oracle on the host ----------------
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(x.to("cpu"))

    print(json.dumps(line), flush=True)

    if args.sweep:
        sweep(g, synth, dev, stream)


def sweep(g, synth, dev, stream):
    """Extra JSON lines: long-context split sweep and batch/group sweep (event medians)."""
    for B in synth.CONFIG4_BATCHES:
        x = synth.config4(B, device=dev)
        nb = kv_bytes(x)
        for ns in synth.CONFIG4_SPLITS:
            ws = g.alloc_workspace(B, 32, 128, ns, dev) if ns > 1 else None
            out = torch.empty_like(x.q)
            f = lambda: g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                       num_splits=ns, scale=x.scale, out=out, workspace=ws)
            for _ in range(3):
                f()
            t = statistics.median(event_times(f, 20, stream))
            print(json.dumps({"sweep": "long-context", "B": B, "T": 32768, "num_splits": ns,
                              "us": round(t * 1e3, 2), "gbs": round(nb / (t * 1e-3) / 1e9, 1)}),
                  flush=True)
        del x
    for hkv in synth.CONFIG5_KV_HEADS:
        for B in synth.CONFIG5_BATCHES:
            x = synth.config5(B, hkv, device=dev)
            nb = kv_bytes(x)
            best = None
            for ns in (1, 2, 4, 8):
                ws = g.alloc_workspace(B, 32, 128, ns, dev) if ns > 1 else None
                out = torch.empty_like(x.q)
                f = lambda: g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table,
                                           x.context_lens, num_splits=ns, scale=x.scale, out=out,
                                           workspace=ws)
                for _ in range(3):
                    f()
                t = statistics.median(event_times(f, 20, stream))
                gbs = nb / (t * 1e-3) / 1e9
                print(json.dumps({"sweep": "batch-group", "B": B, "Hkv": hkv, "T": 1024,
                                  "num_splits": ns, "us": round(t * 1e3, 2), "gbs": round(gbs, 1)}),
                      flush=True)
            del x


if __name__ == "__main__":
    main()
