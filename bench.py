#!/usr/bin/env python3
"""Benchmark of the paged GQA hot path on one MI355X.

A step is one pass of the decode path (the balanced decode kernel, which also
merges the units it cut, ``gqa_decode_paged_balanced``; ``--splits NS`` times the
split path instead) over the paged-decode workload: B=64 sequences, Hq=32, Hkv=8,
D=128, page 16, context lengths uniform in [512, 4096], bf16, pages scattered by a
seeded permutation. Inputs are resident in HBM before the timed region. ``value``
is algorithmic KV bytes (every live K and V row read once) per second of
wall-clock step time; ``roofline.achieved`` uses the GPU time per call from one
HIP event pair on the launch stream around the same timed region.

The same run also reports, each call timed alone after a 1 GiB read that evicts
the L2 caches and the Infinity Cache (median, 10th and 90th percentile): decode
over an E4M3 pool of the same shape; causal prefill (B=4, S=2048, Hq=32, Hkv=8,
D=128, bf16, KV append included) and chunked prefill (4096 cached + 512 new
tokens per sequence) in TFLOP/s of the causal attention flops; the long-context
decode (B in {1, 4, 8}, T=32768) with the balanced partition and NS in
{1, 4, 8, 16}; the batch/group sweep (B in {1..256} x Hkv in {1, 8, 32}, T=1024)
through the balanced entry point; the measured HBM / MFMA ceilings; and the
float64 oracle on the host cores (decode and prefill) as a CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--splits NS]
                       [--no-prefill] [--no-cpu-baseline] [--no-fp8] [--no-sweeps]
                       [--sweep] [--prefill-sweep]
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
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed FMA), TFLOP/s
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


# ---------------- CPU baseline: the float64 oracle in a pool of single-threaded workers --------

_W = {}  # per-worker state of the oracle pool


def _oracle_worker_init(tensors, scale):
    import torch as _t
    _t.set_num_threads(1)
    _W["t"], _W["scale"] = tensors, scale


def _oracle_decode_task(b):
    import oracle  # test infrastructure: the float64 CPU oracle, timed as a baseline only
    q, kc, vc, pt, lens = _W["t"]
    oracle.decode_paged(q[b:b + 1], kc, vc, pt[b:b + 1], lens[b:b + 1], _W["scale"])
    return b


def _oracle_prefill_task(bh):
    import oracle  # test infrastructure: the float64 CPU oracle, timed as a baseline only
    q, k, v = _W["t"]
    oracle.prefill_causal_rows(q, k, v, _W["scale"], [bh])
    return bh


def host_info():
    """CPU model and the cores this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)),
            "os_cpu_count": os.cpu_count()}


def _oracle_pool(tensors, scale):
    """A spawn pool of single-threaded workers (BLAS pinned to one thread each) holding the
    CPU tensors in shared memory; at most 16 workers (one GPU's share of the host)."""
    import torch.multiprocessing as tmp
    n = max(1, min(16, len(os.sched_getaffinity(0))))
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                            "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        pool = tmp.get_context("spawn").Pool(n, initializer=_oracle_worker_init,
                                             initargs=(tensors, scale))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool, n


def cpu_baseline_decode(x_cpu, budget_s=12.0):
    """The float64 oracle over the decode workload, one sequence (all 32 heads) per task,
    whole passes over the batch repeated until ~budget_s of wall time."""
    B = x_cpu.q.shape[0]
    tensors = (x_cpu.q, x_cpu.k_cache, x_cpu.v_cache, x_cpu.page_table, x_cpu.context_lens)
    pool, n = _oracle_pool(tensors, x_cpu.scale)
    try:
        pool.map(_oracle_decode_task, range(min(B, n)))  # workers import the oracle first
        per_seq = [2 * int(x_cpu.context_lens[b]) * x_cpu.k_cache.shape[1] *
                   x_cpu.k_cache.shape[3] * x_cpu.k_cache.element_size() for b in range(B)]
        t0 = time.perf_counter()
        passes = 0
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            pool.map(_oracle_decode_task, range(B), chunksize=1)
            passes += 1
        wall = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    done = passes * sum(per_seq)
    return dict(value=round(done / wall / 1e9, 4), unit="GB/s", cores=n, kind="oracle",
                sample=f"float64 oracle over the whole decode workload ({B} sequences, all "
                       f"32 heads; {sum(per_seq) / 1e6:.0f} MB of KV per pass), {passes} passes "
                       f"in {wall:.1f} s on {n} single-threaded worker processes",
                **host_info())


def cpu_baseline_prefill(p_cpu, budget_s=12.0):
    """The float64 oracle over the causal prefill workload, one (sequence, query head) per
    task; GFLOP/s counts the causal attention flops (the GPU's measure), whole passes repeated
    until ~budget_s."""
    B, S, hq, d = p_cpu.q.shape
    pool, n = _oracle_pool((p_cpu.q, p_cpu.k, p_cpu.v), p_cpu.scale)
    rows = [(b, h) for b in range(B) for h in range(hq)]
    try:
        pool.map(_oracle_prefill_task, rows[:n])
        t0 = time.perf_counter()
        passes = 0
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            pool.map(_oracle_prefill_task, rows, chunksize=1)
            passes += 1
        wall = time.perf_counter() - t0
    finally:
        pool.close()
        pool.join()
    fl = passes * prefill_flops(B, S, hq, d)
    return dict(value=round(fl / wall / 1e9, 2), unit="GFLOP/s", cores=n, kind="oracle",
                sample=f"float64 oracle over the whole causal prefill workload ({B}x{hq} "
                       f"(sequence, head) rows of S={S}), {passes} passes in {wall:.1f} s on "
                       f"{n} single-threaded worker processes; flops counted as the causal "
                       f"half (the oracle itself computes the full score matrix)",
                **host_info())


def percentiles(ts):
    """median, 10th and 90th percentile (ms) of a list of durations."""
    t = sorted(ts)
    q = lambda f: t[min(len(t) - 1, max(0, round(f * (len(t) - 1))))]
    return statistics.median(t), q(0.1), q(0.9)


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
    # equivalent_source_sha: later sources whose build of the counted kernel is the same
    # device assembly (each with the reason), so the counters still describe it
    if h.hexdigest()[:16] not in [rec["source_sha"], *rec.get("equivalent_source_sha", {})]:
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
    ap.add_argument("--no-sweeps", action="store_true",
                    help="leave out the long-context and batch/group legs of the JSON line")
    ap.add_argument("--flushed-calls", type=int, default=20,
                    help="calls timed alone after an L2 / Infinity Cache flush, per leg")
    ap.add_argument("--sweep", action="store_true",
                    help="extra lines: the batch/group sweep under fixed split counts")
    ap.add_argument("--prefill-sweep", action="store_true",
                    help="extra lines: causal prefill over sequence lengths and group sizes")
    ap.add_argument("--lib", default=None,
                    help="load this build of the library instead of gqa_paged_kv_amd/libgqa.so")
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
    g.load(args.lib) if args.lib else g.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # 1 GiB read with ordinary (allocating) loads before each flushed call: evicts the L2s and
    # the Infinity Cache (a streaming read may leave the latter holding the previous call's data)
    scratch = torch.ones(1024 * 2**20 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * 256 * 64, dtype=torch.int32, device=dev)
    flush = lambda: g.bench_flush_read(scratch, sink)
    NF = args.flushed_calls

    def flushed(fn, warm=3):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        return percentiles(event_times(fn, NF, stream, flush=flush))

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
    fmed, fp10, fp90 = flushed(step, warm=0)

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
            "library": os.path.basename(args.lib) if args.lib else "libgqa.so",
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
            "median_us": round(fmed * 1e3, 2), "p10_us": round(fp10 * 1e3, 2),
            "p90_us": round(fp90 * 1e3, 2),
            "gbs": round(nbytes / (fmed * 1e-3) / 1e9, 1),
            "frac": round(nbytes / (fmed * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "note": f"{NF} calls, each after a 1 GiB read with allocating loads (L2 + Infinity Cache evicted)",
        },
    }

    def leg(med, p10, p90, amount, unit_scale, unit, peak):
        rate = amount / (med * 1e-3) / unit_scale
        return {"median_us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2),
                "p90_us": round(p90 * 1e3, 2), "achieved": round(rate, 1), "unit": unit,
                "frac": round(rate / peak, 4)}

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

        r = leg(*flushed(f8step), f8bytes, 1e9, "GB/s", HBM_PEAK_GBS)
        line["decode_fp8"] = {
            "workload": "paged GQA decode, workload 2 shape (B=64, Hq=32, Hkv=8, D=128, page 16, "
                        "T~U[512,4096]) with an E4M3 KV pool (per-tensor scales), bf16 q/out",
            "kv_bytes_per_call": f8bytes, **r,
            "roofline": {"bound": "hbm", "achieved": r["achieved"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": r["frac"],
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

        Bp, S, hq, d = p.q.shape
        fl = prefill_flops(Bp, S, hq, d)
        r = leg(*flushed(pstep), fl, 1e12, "TFLOP/s", BF16_PEAK_TFLOPS)
        line["prefill"] = {
            "workload": "causal GQA prefill, B=4, S=2048, Hq=32, Hkv=8, D=128, bf16, "
                        "append to page-16 cache",
            **r, "tflops": r["achieved"],
            "roofline": {"bound": "mfma", "achieved": r["achieved"], "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["frac"],
                         "traffic": measured_traffic("prefill_causal_bf16_B4_S2048_Hq32_Hkv8"),
                         "kernel": "prefill_causal_kernel<4> (attention + KV append, one launch)"},
            "flops_per_call": fl,
        }
        p_cpu = p.to("cpu") if not args.no_cpu_baseline else None
        del p, pout

        # chunked prefill over a paged context: 4 sequences with 4096 cached tokens each
        # append a 512-token chunk (re-appending the same rows every call is idempotent)
        past, new = [4096] * 4, [512] * 4
        c = synth.chunked_inputs(4, 512, 32, 8, 128, 16, past, new, seed=6000, device=dev)
        cout = torch.empty_like(c.q)

        def cstep():
            g.prefill_paged(c.q, c.k, c.v, c.k_cache, c.v_cache, c.page_table, c.past_lens,
                            c.new_lens, scale=c.scale, out=cout)

        cfl = chunked_flops(past, new, 32, 128)
        r = leg(*flushed(cstep), cfl, 1e12, "TFLOP/s", BF16_PEAK_TFLOPS)
        line["chunked_prefill"] = {
            "workload": "chunked prefill over a paged context, B=4, 4096 cached + 512 new tokens "
                        "per sequence, Hq=32, Hkv=8, D=128, bf16, page 16, permuted pages",
            **r, "tflops": r["achieved"],
            "roofline": {"bound": "mfma", "achieved": r["achieved"], "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": r["frac"],
                         "traffic": measured_traffic("prefill_paged_bf16_B4_P4096_N512_Hq32_Hkv8"),
                         "kernel": "append_at_kernel + prefill_causal_kernel<4, paged> (one call)"},
            "flops_per_call": cfl,
        }
        del c, cout

    # ---------------- long-context split-K decode and the batch / group sweep ----------------
    if not args.no_sweeps:
        lc = []
        for Bl in synth.CONFIG4_BATCHES:
            xl = synth.config4(Bl, device=dev)
            nb = kv_bytes(xl)
            lout = torch.empty_like(xl.q)
            bws = g.balanced_workspace(Bl, 32, 8, 128, dev)
            fn = lambda: g.decode_paged_balanced(xl.q, xl.k_cache, xl.v_cache, xl.page_table,
                                                 xl.context_lens, scale=xl.scale, out=lout,
                                                 workspace=bws)
            lc.append({"B": Bl, "partition": "balanced",
                       **leg(*flushed(fn), nb, 1e9, "GB/s", HBM_PEAK_GBS)})
            for nsl in synth.CONFIG4_SPLITS:
                sws = g.alloc_workspace(Bl, 32, 128, nsl, dev) if nsl > 1 else None
                fn = lambda: g.decode_paged(xl.q, xl.k_cache, xl.v_cache, xl.page_table,
                                            xl.context_lens, num_splits=nsl, scale=xl.scale,
                                            out=lout, workspace=sws)
                lc.append({"B": Bl, "num_splits": nsl,
                           **leg(*flushed(fn), nb, 1e9, "GB/s", HBM_PEAK_GBS)})
            del xl, lout, bws
        line["long_context"] = {
            "workload": "long-context decode, T=32768, Hq=32, Hkv=8, D=128, bf16, page 16, "
                        "64 hot keys x4 per sequence; decode + combine per call",
            "points": lc}
        bg = []
        for hkv in synth.CONFIG5_KV_HEADS:
            for Bs in synth.CONFIG5_BATCHES:
                xs = synth.config5(Bs, hkv, device=dev)
                nb = kv_bytes(xs)
                sout = torch.empty_like(xs.q)
                bws = g.balanced_workspace(Bs, 32, hkv, 128, dev)
                fn = lambda: g.decode_paged_balanced(xs.q, xs.k_cache, xs.v_cache,
                                                     xs.page_table, xs.context_lens,
                                                     scale=xs.scale, out=sout, workspace=bws)
                route = g.balanced_route(Bs, 32, hkv, 128, xs.page_table.shape[1])
                med, p10, p90 = flushed(fn)
                pt_ = {"B": Bs, "Hkv": hkv, "G": 32 // hkv,
                       "route": "persistent" if route == 0 else f"split NS={route}",
                       **leg(med, p10, p90, nb, 1e9, "GB/s", HBM_PEAK_GBS)}
                if hkv == 1:  # MQA: 4*D flop per (token, query head) on the vector ALU bound
                    fl = 4.0 * 128 * int(xs.context_lens.sum()) * 32
                    pt_["valu_frac"] = round(fl / (med * 1e-3) / 1e12 / FP32_VALU_PEAK_TFLOPS, 4)
                    if Bs == 256:
                        pt_["traffic"] = measured_traffic("decode_mq_bf16_B256_Hq32_Hkv1_T1024")
                        pt_["kernel"] = "decode_mq_kernel<128,32> (matrix-core scores and PV)"
                bg.append(pt_)
                del xs, sout, bws
        line["batch_group"] = {
            "workload": "batch/group sweep decode, T=1024, Hq=32, D=128, bf16, page 16, "
                        "through gqa_decode_paged_balanced (the library's route)",
            "points": bg}

    ceil = ceilings(g, dev, stream)
    line["measured_ceiling"] = dict(ceil, decode_frac_of_read=round(achieved / ceil["stream_read_gbs"], 4))
    for key in ("prefill", "chunked_prefill"):
        if key in line:
            line[key]["frac_of_mfma_ceiling"] = round(line[key]["tflops"] / ceil["mfma_bf16_tflops"], 4)
    del scratch

    # ---------------- CPU baseline: the float64 oracle on the host ----------------
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(x.to("cpu"))
        if not args.no_prefill:
            line["cpu_baseline_prefill"] = cpu_baseline_prefill(p_cpu)

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
    """Extra JSON lines: the batch/group sweep under fixed split counts (split path, NS in
    {1, 2, 4, 8}) next to the library's route. Every call is timed alone with HIP events after
    a 1 GiB read with allocating loads that evicts the L2 and the Infinity Cache; median and 10th / 90th
    percentile of 20 calls."""
    scratch = torch.ones(1024 * 2**20 // 4, dtype=torch.float32, device=dev)
    sink = torch.empty(4 * 256 * 64, dtype=torch.int32, device=dev)
    flush = lambda: g.bench_flush_read(scratch, sink)

    def timed(f, nb, **fields):
        for _ in range(3):
            f()
        med, p10, p90 = percentiles(event_times(f, 20, stream, flush=flush))
        print(json.dumps({**fields, "us": round(med * 1e3, 2), "p10_us": round(p10 * 1e3, 2),
                          "p90_us": round(p90 * 1e3, 2),
                          "gbs": round(nb / (med * 1e-3) / 1e9, 1)}), flush=True)

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
