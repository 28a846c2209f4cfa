#!/usr/bin/env python3
"""Benchmark of the paged GQA hot path on one MI355X.

A step is one pass of the decode path (the balanced decode kernel, which also
merges the units it cut, ``gqa_decode_paged_balanced``; ``--splits NS`` times the
split path instead) over
the paged-decode workload: B=64 sequences, Hq=32, Hkv=8, D=128, page 16, context
lengths uniform in [512, 4096], bf16, pages scattered by a seeded
permutation. Inputs are resident in HBM before the timed region. ``value`` is
algorithmic KV bytes (every live K and V row read once) per second of
wall-clock step time; ``roofline.achieved`` uses the GPU time per call from one
HIP event pair on the launch stream around the same timed region. The same run
also times decode over an E4M3 pool of the same shape, causal prefill (B=4,
S=2048, Hq=32, Hkv=8, D=128, bf16, KV append included) and chunked prefill
(4096 cached + 512 new tokens per sequence), reporting TFLOP/s for the causal
attention flops, plus the float64 oracle on the host cores as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--splits NS]
                       [--no-prefill] [--no-cpu-baseline] [--no-fp8] [--sweep]
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
DEFAULT_SPLITS = 0  # balanced partition (gqa_decode_paged_balanced)


def kv_bytes(x) -> int:
    """Algorithmic bytes of one decode pass: every live K and V row once."""
    T = int(x.context_lens.sum())
    hkv, d = x.k_cache.shape[1], x.k_cache.shape[3]
    return 2 * T * hkv * d * x.k_cache.element_size()


def prefill_flops(B, S, hq, d) -> float:
    """QK^T and PV flops of the causal half: 4*D*S(S+1)/2 per (b, head)."""
    return 4.0 * d * S * (S + 1) / 2 * B * hq


def chunked_flops(past, new, hq, d) -> float:
    """QK^T and PV flops of chunked prefill: new row i attends past + i + 1 keys, so
    4*D*(n*p + n(n+1)/2) per (b, head); ``past`` / ``new`` are per-sequence lists."""
    return sum(4.0 * d * (n * p + n * (n + 1) / 2) * hq for p, n in zip(past, new))


def event_times_queued(fn, n, stream):
    """Per-call durations (ms) from HIP events around each of n calls enqueued back to back
    (no host synchronisation in between, so the GPU never waits for the host)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def event_times(fn, n, stream, flush=None):
    """Per-call durations (ms) from HIP events recorded on ``stream``, each call run alone
    (after ``flush`` if given)."""
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
    """The float64 oracle over the decode workload's sequences, repeated until ~budget_s."""
    import oracle  # test infrastructure: the float64 CPU oracle, timed as a baseline only
    B = x_cpu.q.shape[0]
    t0w, t0c = time.perf_counter(), time.process_time()
    done_bytes = 0
    n = 0
    while time.perf_counter() - t0w < budget_s:
        b = n % B
        T = int(x_cpu.context_lens[b])
        oracle.decode_paged(x_cpu.q[b:b + 1], x_cpu.k_cache, x_cpu.v_cache,
                            x_cpu.page_table[b:b + 1], x_cpu.context_lens[b:b + 1], x_cpu.scale)
        done_bytes += 2 * T * x_cpu.k_cache.shape[1] * x_cpu.k_cache.shape[3] * 2
        n += 1
    wall = time.perf_counter() - t0w
    cpu = time.process_time() - t0c
    return dict(value=round(done_bytes / wall / 1e9, 4), unit="GB/s",
                cores=max(1, round(cpu / wall)), kind="oracle",
                sample=f"float64 oracle, {n} sequence decodes of the decode workload "
                       f"(all 32 heads each; {done_bytes / 1e6:.0f} MB of KV) in {wall:.1f} s",
                host_cores=len(os.sched_getaffinity(0)))


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gqa_paged_kv_amd", "csrc")


def measured_traffic(key):
    """HBM bytes per call from the committed rocprofv3 PMC summary, or None if the kernel
    sources changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(PROFILES, "traffic.json")))[key]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(CSRC, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    if h.hexdigest()[:16] != rec["source_sha"]:
        return None
    return round(rec["hbm_bytes_per_call"])


def ceilings(g, dev, stream):
    """What this GPU reaches: a 2 GiB streaming read and a bf16 MFMA-only loop."""
    src = torch.ones(2 * 2**30 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * 256 * 64, dtype=torch.int32, device=dev)
    f = lambda: g.bench_stream_read(src, sink, 8, 1)
    f()
    t_read = statistics.median(event_times(f, 10, stream))
    del src
    # a plain device copy of known size (512 MiB read + 512 MiB written): the reference that
    # calibrates the rocprofv3 FETCH_SIZE / WRITE_SIZE counters
    a = torch.empty(2**27, dtype=torch.float32, device=dev)
    a_copy = torch.empty_like(a)
    a_copy.copy_(a)
    del a, a_copy
    fs = torch.empty(1024 * 8, dtype=torch.float32, device=dev)
    blocks, iters = 1024, 4096
    h = lambda: g.bench_mfma_bf16(fs, blocks, iters)
    h()
    t_mfma = statistics.median(event_times(h, 5, stream))
    return {"stream_read_gbs": round(2 * 2**30 / (t_read * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(blocks * 8 * iters * 32768 / (t_mfma * 1e-3) / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--splits", type=int, default=DEFAULT_SPLITS)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="extra lines for the split/batch sweeps")
    ap.add_argument("--prefill-sweep", action="store_true",
                    help="extra lines: causal prefill over sequence lengths and group sizes")
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
    ns = args.splits  # 0: the library's balanced partition
    out = torch.empty_like(x.q)
    B, Hq, D = x.q.shape
    Hkv = x.k_cache.shape[1]
    if ns > 0:
        ws = g.alloc_workspace(B, Hq, D, ns, dev) if ns > 1 else None
    else:
        ws = g.balanced_workspace(B, Hq, Hkv, D, dev)
    nbytes = kv_bytes(x)

    def step():
        if ns > 0:
            g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                           num_splits=ns, scale=x.scale, out=out, workspace=ws)
        else:
            g.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                    scale=x.scale, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    # Timed region: K calls enqueued back to back, one HIP event pair on the launch stream
    # around the whole region (per-call events would add their own gaps to the stream).
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    ev_avg = t_begin.elapsed_time(t_end) / args.steps  # GPU time per call in the region
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (ev_avg * 1e-3) / 1e9
    # per-call durations (events around each call) as a cross-check
    ev_call = statistics.fmean(event_times_queued(step, 100, stream))

    # same launch preceded by a 1 GiB read that evicts L2 and the Infinity Cache
    scratch = torch.ones(1024 * 2**20 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * 256 * 64, dtype=torch.int32, device=dev)
    flushed = event_times(step, 30, stream,
                          flush=lambda: g.bench_stream_read(scratch, sink, 8, 1))
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
            "partition": "balanced (equal page shares per wave)" if ns == 0 else f"{ns} splits",
            "kv_bytes_per_step": nbytes,
            "total_context_tokens": int(x.context_lens.sum()),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_balanced_bf16_B64_Hq32_Hkv8") if ns == 0 else None,
            "traffic_unit": "HBM bytes per call (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, calibrated)",
            "kernel": ("balanced_kernel<bf16,128,4> (one decode call, one launch)" if ns == 0
                       else "decode_regs_kernel<bf16,128,4> + combine_kernel (one decode call)"),
            "event_avg_us": round(ev_avg * 1e3, 2),
            "event_per_call_us": round(ev_call * 1e3, 2),
        },
        "decode_flushed": {
            "median_us": round(flushed_med * 1e3, 2),
            "gbs": round(nbytes / (flushed_med * 1e-3) / 1e9, 1),
            "frac": round(nbytes / (flushed_med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": "each launch preceded by a 1 GiB streaming read (L2 + Infinity Cache evicted)",
        },
    }
    del scratch

    # ---------------- decode over an 8-bit KV pool (workload 2, E4M3) ----------------
    if not args.no_fp8:
        f8 = synth.config2_fp8("e4m3", device=dev)
        f8out = torch.empty_like(f8.q)
        f8ws = g.balanced_workspace(B, Hq, Hkv, D, dev)
        f8bytes = int(f8.context_lens.sum()) * Hkv * D * 1 * 2

        def f8step():
            g.decode_paged_fp8(f8.q, f8.k_cache, f8.v_cache, f8.k_scale, f8.v_scale,
                               f8.page_table, f8.context_lens, fmt="e4m3", scale=f8.scale,
                               out=f8out, workspace=f8ws)

        for _ in range(10):
            f8step()
        torch.cuda.synchronize()
        f8med = statistics.median(event_times_queued(f8step, 100, stream))
        f8gbs = f8bytes / (f8med * 1e-3) / 1e9
        line["decode_fp8"] = {
            "workload": "paged GQA decode, workload 2 shape (B=64, Hq=32, Hkv=8, D=128, page 16, "
                        "T~U[512,4096]) with an E4M3 KV pool (per-tensor scales), bf16 q/out",
            "kv_bytes_per_call": f8bytes,
            "median_us": round(f8med * 1e3, 2),
            "gbs": round(f8gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(f8gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(f8gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_balanced_fp8e4m3_B64_Hq32_Hkv8"),
                         "kernel": "balanced_kernel<bf16,128,4,fp8e4m3> (one launch)"},
        }
        del f8, f8out, f8ws

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
        pt = event_times_queued(pstep, 30, stream)
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
                         "traffic": measured_traffic("prefill_causal_bf16_B4_S2048_Hq32_Hkv8"),
                         "kernel": "prefill_causal_kernel<4> (attention + KV append, one launch)"},
            "flops_per_call": fl,
        }
        del p, pout

        # chunked prefill over a paged context: 4 sequences with 4096 cached tokens each
        # append a 512-token chunk (re-appending the same rows every call is idempotent)
        past, new = [4096] * 4, [512] * 4
        c = synth.chunked_inputs(4, 512, 32, 8, 128, 16, past, new, seed=6000, device=dev)
        cout = torch.empty_like(c.q)

        def cstep():
            g.prefill_paged(c.q, c.k, c.v, c.k_cache, c.v_cache, c.page_table, c.past_lens,
                            c.new_lens, scale=c.scale, out=cout)

        for _ in range(5):
            cstep()
        torch.cuda.synchronize()
        cmed = statistics.median(event_times_queued(cstep, 30, stream))
        cfl = chunked_flops(past, new, 32, 128)
        ctf = cfl / (cmed * 1e-3) / 1e12
        line["chunked_prefill"] = {
            "workload": "chunked prefill over a paged context, B=4, 4096 cached + 512 new tokens "
                        "per sequence, Hq=32, Hkv=8, D=128, bf16, page 16, permuted pages",
            "median_us": round(cmed * 1e3, 2),
            "tflops": round(ctf, 1),
            "roofline": {"bound": "mfma", "achieved": round(ctf, 1), "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ctf / BF16_PEAK_TFLOPS, 4),
                         "traffic": measured_traffic("prefill_paged_bf16_B4_P4096_N512_Hq32_Hkv8"),
                         "kernel": "append_at_kernel + prefill_causal_kernel<4, paged> (one call)"},
            "flops_per_call": cfl,
        }
        del c, cout

    ceil = ceilings(g, dev, stream)
    line["measured_ceiling"] = dict(ceil, decode_frac_of_read=round(achieved / ceil["stream_read_gbs"], 4))
    for key in ("prefill", "chunked_prefill"):
        if key in line:
            line[key]["frac_of_mfma_ceiling"] = round(line[key]["tflops"] / ceil["mfma_bf16_tflops"], 4)

    # ---------------- CPU baseline: the float64 oracle on the host ----------------
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(x.to("cpu"))

    print(json.dumps(line), flush=True)

    if args.sweep:
        sweep(g, synth, dev, stream)
    if args.prefill_sweep:
        prefill_sweep(g, synth, dev, stream)


def prefill_sweep(g, synth, dev, stream):
    """Extra JSON lines: causal prefill (bf16, D=128, KV append included) over sequence lengths
    at the benchmark's heads (Hq=32, Hkv=8; B*S = 8192 tokens) and over group sizes at S=2048
    (Hq=32, Hkv = 32, 16, 8, 4; B=4). Median of 30 calls timed back to back with HIP events."""
    shapes = [(16, 512, 32, 8), (8, 1024, 32, 8), (4, 2048, 32, 8), (2, 4096, 32, 8),
              (1, 8192, 32, 8), (4, 2048, 32, 32), (4, 2048, 32, 16), (4, 2048, 32, 4)]
    for B, S, hq, hkv in shapes:
        p = synth.prefill_inputs(B, S, hq, hkv, 128, 16, seed=B * S + hkv, device=dev)
        out = torch.empty_like(p.q)

        def step():
            g.prefill_causal(p.q, p.k, p.v, p.k_cache, p.v_cache, p.page_table, scale=p.scale,
                             out=out)

        for _ in range(5):
            step()
        torch.cuda.synchronize()
        med = statistics.median(event_times_queued(step, 30, stream))
        fl = prefill_flops(B, S, hq, 128)
        print(json.dumps({"prefill_sweep": f"B={B} S={S} Hq={hq} Hkv={hkv} G={hq // hkv}",
                          "us": round(med * 1e3, 2),
                          "tflops": round(fl / (med * 1e-3) / 1e12, 1),
                          "frac": round(fl / (med * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}), flush=True)
        del p, out


def sweep(g, synth, dev, stream):
    """Extra JSON lines: long-context split sweep and batch/group sweep. Every call is timed
    alone with HIP events after a 1 GiB streaming read that evicts the L2 and the Infinity
    Cache (the long-context B=1 pool, 134 MB, would otherwise stay in the 256 MB cache);
    median and 10th / 90th percentile of 20 calls."""
    scratch = torch.ones(1024 * 2**20 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * 256 * 64, dtype=torch.int32, device=dev)
    flush = lambda: g.bench_stream_read(scratch, sink, 8, 1)

    def timed(f, nb, **fields):
        for _ in range(3):
            f()
        ts = sorted(event_times(f, 20, stream, flush=flush))
        t = statistics.median(ts)
        print(json.dumps({**fields, "us": round(t * 1e3, 2), "p10_us": round(ts[2] * 1e3, 2),
                          "p90_us": round(ts[17] * 1e3, 2),
                          "gbs": round(nb / (t * 1e-3) / 1e9, 1)}), flush=True)

    for B in synth.CONFIG4_BATCHES:
        x = synth.config4(B, device=dev)
        nb = kv_bytes(x)
        bws = g.balanced_workspace(B, 32, 8, 128, dev)
        out = torch.empty_like(x.q)
        timed(lambda: g.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table,
                                              x.context_lens, scale=x.scale, out=out,
                                              workspace=bws),
              nb, sweep="long-context", B=B, T=32768, partition="balanced")
        for ns in synth.CONFIG4_SPLITS:
            ws = g.alloc_workspace(B, 32, 128, ns, dev) if ns > 1 else None
            timed(lambda: g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table,
                                         x.context_lens, num_splits=ns, scale=x.scale, out=out,
                                         workspace=ws),
                  nb, sweep="long-context", B=B, T=32768, num_splits=ns)
        del x
    for hkv in synth.CONFIG5_KV_HEADS:
        for B in synth.CONFIG5_BATCHES:
            x = synth.config5(B, hkv, device=dev)
            nb = kv_bytes(x)
            bws = g.balanced_workspace(B, 32, hkv, 128, dev)
            out = torch.empty_like(x.q)
            timed(lambda: g.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table,
                                                  x.context_lens, scale=x.scale, out=out,
                                                  workspace=bws),
                  nb, sweep="batch-group", B=B, Hkv=hkv, T=1024, partition="balanced")
            for ns in (1, 2, 4, 8):
                ws = g.alloc_workspace(B, 32, 128, ns, dev) if ns > 1 else None
                timed(lambda: g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table,
                                             x.context_lens, num_splits=ns, scale=x.scale,
                                             out=out, workspace=ws),
                      nb, sweep="batch-group", B=B, Hkv=hkv, T=1024, num_splits=ns)
            del x
    del scratch, sink


if __name__ == "__main__":
    main()
