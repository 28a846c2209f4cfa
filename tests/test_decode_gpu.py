"""GPU parity of paged GQA decode, split/combine and gather against the float64 oracle.

Every case is seeded and synthetic (synth/); the oracle runs on the CPU on the
same tensors the kernels read.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import assert_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _sync():
    torch.cuda.synchronize()


def _ref(x):
    c = x.to("cpu")
    return oracle.decode_paged(c.q, c.k_cache, c.v_cache, c.page_table, c.context_lens, c.scale)


def _run(g, x, ns=1):
    out = g.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, num_splits=ns,
                         scale=x.scale)
    _sync()
    return out


# ---------------------------------------------------------------- workload 1

@pytest.mark.parametrize("ns", [1, 2, 4, 16])
def test_config1_tiny_fp32(gpu_lib, ns):
    print(f"[decode] config1 fp32 ns={ns}", flush=True)
    x = synth.config1(device=DEV)
    out = _run(gpu_lib, x, ns)
    assert_close(out, _ref(x), "f32", f"config1 ns={ns}")


# ---------------------------------------------------- small shapes, every instance

SMALL = [
    # dtype, D, Hq, Hkv, lens
    ("bf16", 128, 8, 2, [1, 77, 300]),
    ("bf16", 128, 32, 8, [16, 64, 65, 129]),
    ("bf16", 128, 4, 4, [5, 200]),
    ("bf16", 128, 32, 1, [63, 190]),
    ("bf16", 128, 32, 2, [33, 250]),
    ("bf16", 128, 16, 2, [100]),
    ("bf16", 64, 8, 2, [1, 130, 257]),
    ("bf16", 64, 32, 1, [77, 511]),
    ("bf16", 64, 16, 1, [40]),
    ("f32", 64, 8, 2, [1, 100, 255]),
    ("f32", 64, 32, 1, [31, 97]),
    ("f32", 128, 8, 2, [3, 33, 150]),
    ("f32", 128, 32, 4, [70]),
    ("f32", 128, 16, 1, [45, 46]),
    ("f32", 64, 2, 1, [18]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}-D{c[1]}-{c[2]}x{c[3]}")
@pytest.mark.parametrize("ns", [1, 3])
def test_small_shapes(gpu_lib, case, ns):
    dtype, D, hq, hkv, lens = case
    print(f"[decode] small {case} ns={ns}", flush=True)
    x = synth.decode_inputs(len(lens), hq, hkv, D, 16, lens, dtype,
                            seed=D + 7 * hq + 13 * hkv + len(lens), device=DEV)
    out = _run(gpu_lib, x, ns)
    assert_close(out, _ref(x), dtype, f"{case} ns={ns}")


def test_empty_and_single_token_sequences(gpu_lib):
    print("[decode] empty/single", flush=True)
    x = synth.decode_inputs(4, 8, 2, 128, 16, [0, 1, 0, 17], "bf16", seed=5, device=DEV)
    for ns in (1, 4):
        out = _run(gpu_lib, x, ns)
        assert torch.all(out[0] == 0) and torch.all(out[2] == 0)
        ref = _ref(x)
        # one token: the output is exactly that token's V row (rounded to bf16 it is itself)
        pt = x.page_table.cpu()
        v0 = x.v_cache[int(pt[1, 0]), :, 0].cpu()
        assert torch.equal(out[1].cpu(), v0.repeat_interleave(4, 0))
        assert_close(out, ref, "bf16", f"empty/single ns={ns}")


def test_context_longer_than_table_is_clamped(gpu_lib):
    print("[decode] clamp", flush=True)
    x = synth.decode_inputs(2, 8, 2, 128, 16, [40, 64], "bf16", seed=6, device=DEV)
    lens_big = torch.tensor([40, 10_000], dtype=torch.int32, device=DEV)  # row 1 table holds 4 pages
    out = gpu_lib.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, lens_big, scale=x.scale)
    _sync()
    ref = _ref(x)  # T_1 = 64 = max_pages * P
    assert_close(out, ref, "bf16", "clamped")


# ---------------------------------------------------------------- workload 2

@pytest.fixture(scope="module")
def cfg2():
    x = synth.config2(device=DEV)
    return x, _ref(x)


@pytest.mark.parametrize("ns", [1, 4, 8, 16])
def test_config2_paged_bf16(gpu_lib, cfg2, ns):
    print(f"[decode] config2 ns={ns}", flush=True)
    x, ref = cfg2
    out = _run(gpu_lib, x, ns)
    assert_close(out, ref, "bf16", f"config2 ns={ns}")


def test_config2_deterministic_and_page_permutation_invariant(gpu_lib, cfg2):
    print("[decode] config2 determinism / permutation", flush=True)
    x, _ = cfg2
    a = _run(gpu_lib, x, 8)
    b = _run(gpu_lib, x, 8)
    assert torch.equal(a, b)
    n = x.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(77)).to(DEV)
    k2 = torch.empty_like(x.k_cache)
    v2 = torch.empty_like(x.v_cache)
    k2[perm] = x.k_cache
    v2[perm] = x.v_cache
    pt2 = x.page_table.clone()
    live = pt2 >= 0
    pt2[live] = perm[pt2[live].long()].to(torch.int32)
    for ns in (1, 8):
        base = _run(gpu_lib, x, ns)
        moved = gpu_lib.decode_paged(x.q, k2, v2, pt2, x.context_lens, num_splits=ns, scale=x.scale)
        _sync()
        assert torch.equal(base, moved), f"ns={ns}"


def test_poison_does_not_leak(gpu_lib):
    print("[decode] poison", flush=True)
    x = synth.decode_inputs(3, 32, 8, 128, 16, [37, 300, 16], "bf16", seed=8, device=DEV,
                            poison=True)
    clean_k = torch.nan_to_num(x.k_cache, nan=0.0)
    clean_v = torch.nan_to_num(x.v_cache, nan=0.0)
    pt_far = x.page_table.clone()
    pt_far[pt_far < 0] = 2**30  # entries past the last page: never read
    for ns in (1, 3):
        a = _run(gpu_lib, x, ns)
        b = gpu_lib.decode_paged(x.q, clean_k, clean_v, pt_far, x.context_lens, num_splits=ns,
                                 scale=x.scale)
        _sync()
        assert torch.isfinite(a.float()).all()
        assert torch.equal(a, b), f"ns={ns}"


# ---------------------------------------------------------------- workload 4

@pytest.mark.parametrize("B", synth.CONFIG4_BATCHES)
def test_config4_long_context_splits(gpu_lib, B):
    print(f"[decode] config4 B={B}", flush=True)
    x = synth.config4(B, device=DEV)
    ref = _ref(x)
    outs = {}
    for ns in synth.CONFIG4_SPLITS:
        outs[ns] = _run(gpu_lib, x, ns)
        assert_close(outs[ns], ref, "bf16", f"config4 B={B} ns={ns}")


# ---------------------------------------------------------------- workload 5

@pytest.mark.parametrize("Hkv", synth.CONFIG5_KV_HEADS)
@pytest.mark.parametrize("B", synth.CONFIG5_BATCHES)
def test_config5_sweep_whole_output(gpu_lib, B, Hkv):
    """Every (B, Hkv) point of the batch/group sweep: all B x 32 output rows against the
    float64 oracle, on the split path (one split) and through the balanced entry point (the
    route the benchmark times)."""
    print(f"[decode] config5 B={B} Hkv={Hkv}", flush=True)
    x = synth.config5(B, Hkv, device=DEV)
    ref = _ref(x)
    assert_close(_run(gpu_lib, x, 1), ref, "bf16", f"config5 B={B} Hkv={Hkv} split")
    assert_close(_run_bal(gpu_lib, x), ref, "bf16", f"config5 B={B} Hkv={Hkv} balanced")
    del x


# ---------------------------------------------------------------- gather / combine

@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_gather_is_bit_exact(gpu_lib, dtype, D):
    print(f"[gather] {dtype} D={D}", flush=True)
    x = synth.decode_inputs(3, 8, 4, D, 16, [5, 48, 131], dtype, seed=9, device=DEV)
    dst = gpu_lib.gather_paged(x.k_cache, x.page_table, x.context_lens)
    _sync()
    c = x.to("cpu")
    want = oracle.gather_paged(c.k_cache, c.page_table, c.context_lens, 16)
    dst = dst.cpu()
    for b in range(3):
        T = int(c.context_lens[b])
        assert torch.equal(dst[b, :T].view(torch.int16 if dtype == "bf16" else torch.int32),
                           want[b].view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_combine_standalone(gpu_lib, out_dtype):
    print(f"[combine] {out_dtype}", flush=True)
    g = torch.Generator().manual_seed(3)
    B, Hq, NS, D = 3, 8, 6, 128
    o = torch.randn(B, Hq, NS, D, generator=g)
    lse = torch.randn(B, Hq, NS, generator=g) * 5
    lse[0, 0, :] = -float("inf")         # all splits empty -> zero
    lse[0, 1, 1:] = -float("inf")        # one live split
    lse[1, 2, 3] = 80.0                  # one dominant split
    lse[2, :, ::2] = -float("inf")       # empty splits interleaved
    out = gpu_lib.combine_splits(o.to(DEV), lse.to(DEV), out_dtype)
    _sync()
    ref = oracle.combine_splits(o, lse)
    assert torch.all(out[0, 0] == 0)
    assert_close(out, ref, "f32" if out_dtype == torch.float32 else "bf16", "combine")


# ---------------------------------------------------------------- balanced partition

def _run_bal(g, x):
    out = g.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                  scale=x.scale)
    _sync()
    return out


def _route_table(route, B, hq, hkv, lens):
    """Page-table width that sends a balanced call down `route`: "split" keeps the narrowest
    table (small problems take the split path), "persistent" widens it past the small-problem
    limits ((sequence, KV head, page) items: 65,536 for G = 1, 16,384 for G = 2, 8,192 for
    G = 4, 1,024 for G = 8)."""
    if route == "split":
        return None
    limit = {1: 65536, 2: 16384, 4: 8192}.get(hq // hkv, 1024)
    return max(max((t + 15) // 16 for t in lens), 1, limit // (B * hkv) + 1)


def _bal_inputs(g, route, B, hq, hkv, D, lens, dtype, seed, **kw):
    x = synth.decode_inputs(B, hq, hkv, D, 16, lens, dtype, seed=seed, device=DEV,
                            max_pages=_route_table(route, B, hq, hkv, lens), **kw)
    r = g.balanced_route(B, hq, hkv, D, x.page_table.shape[1])
    assert (r == 0) == (route == "persistent"), f"route {r} for a {route} case"
    return x


# the persistent kernel serves G <= 8 only
BAL_CASES = [(c, r) for c in SMALL for r in ("split", "persistent")
             if r == "split" or c[2] // c[3] <= 8]


@pytest.mark.parametrize("case,route", BAL_CASES,
                         ids=lambda c: c if isinstance(c, str) else f"{c[0]}-D{c[1]}-{c[2]}x{c[3]}")
def test_balanced_small_shapes(gpu_lib, case, route):
    dtype, D, hq, hkv, lens = case
    print(f"[balanced] small {case} {route}", flush=True)
    x = _bal_inputs(gpu_lib, route, len(lens), hq, hkv, D, lens, dtype,
                    seed=D + 7 * hq + 13 * hkv + len(lens))
    assert_close(_run_bal(gpu_lib, x), _ref(x), dtype, f"balanced {case} {route}")


@pytest.mark.parametrize("route", ["split", "persistent"])
def test_balanced_config1_and_empty_sequences(gpu_lib, route):
    print(f"[balanced] config1 / empty {route}", flush=True)
    # workload 1's inputs, in a page table as wide as the route needs
    x = synth.config1(device=DEV, max_pages=_route_table(route, 2, 8, 2, [256, 256]))
    r = gpu_lib.balanced_route(2, 8, 2, 64, x.page_table.shape[1])
    assert (r == 0) == (route == "persistent")
    assert_close(_run_bal(gpu_lib, x), _ref(x), "f32", f"balanced config1 {route}")
    y = _bal_inputs(gpu_lib, route, 5, 8, 2, 128, [0, 1, 0, 17, 0], "bf16", seed=5)
    out = torch.full_like(y.q, float("nan"))
    gpu_lib.decode_paged_balanced(y.q, y.k_cache, y.v_cache, y.page_table, y.context_lens,
                                  scale=y.scale, out=out)
    _sync()
    for b in (0, 2, 4):
        assert torch.all(out[b] == 0)
    assert_close(out, _ref(y), "bf16", f"balanced empty {route}")


# The persistent kernel walks 16- and 32-bit caches kv-head-major: a share runs through the
# sequences of one kv head, skipping empty ones, and wraps to the first non-empty sequence of
# the next kv head; the resident waves are rounded down to a multiple of Hkv. Batches of more
# than 64 sequences (the start-up scan's chunk), empty sequences at both ends and in runs, and
# kv-head counts that do not divide the wave count.
def _walk_lens(B, seed):
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, 700, (B,), generator=g)
    for i in (0, 1, B // 2, B // 2 + 1, B // 2 + 2, B - 2, B - 1):
        lens[i] = 0
    return [int(t) for t in lens]


WALK_CASES = [
    ("bf16", 128, 32, 8, 100),
    ("bf16", 128, 12, 3, 70),
    ("bf16", 64, 10, 5, 67),
    ("f32", 128, 16, 4, 66),
]


@pytest.mark.parametrize("case", WALK_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-{c[2]}x{c[3]}-B{c[4]}")
def test_balanced_kv_head_major_walk(gpu_lib, case):
    dtype, D, hq, hkv, B = case
    print(f"[balanced] kv-head-major walk {case}", flush=True)
    lens = _walk_lens(B, seed=B + hkv)
    x = _bal_inputs(gpu_lib, "persistent", B, hq, hkv, D, lens, dtype, seed=3 * B + hq)
    out = _run_bal(gpu_lib, x)
    assert_close(out, _ref(x), dtype, f"balanced walk {case}")
    again = _run_bal(gpu_lib, x)
    assert torch.equal(out, again), "a second call differs"


def test_balanced_config2_parity_determinism_permutation(gpu_lib, cfg2):
    print("[balanced] config2", flush=True)
    x, ref = cfg2
    a = _run_bal(gpu_lib, x)
    assert_close(a, ref, "bf16", "balanced config2")
    assert torch.equal(a, _run_bal(gpu_lib, x))
    n = x.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(78)).to(DEV)
    k2 = torch.empty_like(x.k_cache)
    v2 = torch.empty_like(x.v_cache)
    k2[perm] = x.k_cache
    v2[perm] = x.v_cache
    pt2 = x.page_table.clone()
    live = pt2 >= 0
    pt2[live] = perm[pt2[live].long()].to(torch.int32)
    moved = gpu_lib.decode_paged_balanced(x.q, k2, v2, pt2, x.context_lens, scale=x.scale)
    _sync()
    assert torch.equal(a, moved)


@pytest.mark.parametrize("route", ["split", "persistent"])
def test_balanced_poison(gpu_lib, route):
    print(f"[balanced] poison {route}", flush=True)
    x = _bal_inputs(gpu_lib, route, 3, 32, 8, 128, [37, 300, 16], "bf16", seed=8)
    clean_k = torch.nan_to_num(x.k_cache, nan=0.0)
    clean_v = torch.nan_to_num(x.v_cache, nan=0.0)
    pt_far = x.page_table.clone()
    pt_far[pt_far < 0] = 2**30
    a = _run_bal(gpu_lib, x)
    b = gpu_lib.decode_paged_balanced(x.q, clean_k, clean_v, pt_far, x.context_lens, scale=x.scale)
    _sync()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("B", synth.CONFIG4_BATCHES)
def test_balanced_config4(gpu_lib, B):
    print(f"[balanced] config4 B={B}", flush=True)
    x = synth.config4(B, device=DEV)
    assert_close(_run_bal(gpu_lib, x), _ref(x), "bf16", f"balanced config4 B={B}")


@pytest.mark.parametrize("B,hq,hkv,T", [(1, 32, 8, 1024), (1, 32, 32, 1024), (2, 8, 2, 100),
                                         (1, 4, 1, 16), (3, 32, 8, 40)])
def test_balanced_small_batches_use_fewer_waves(gpu_lib, B, hq, hkv, T):
    """Persistent kernel on batches with fewer than a few pages per resident wave: only N / 4
    waves take a share (the others must return at once) and the merge of cut units uses the
    same partition (the page table is widened so that the balanced entry point does not
    hand these small problems to the split path)."""
    print(f"[balanced] small batch B={B} {hq}x{hkv} T={T}", flush=True)
    x = _bal_inputs(gpu_lib, "persistent", B, hq, hkv, 128, [T] * B, "bf16", seed=B * 31 + T)
    assert_close(_run_bal(gpu_lib, x), _ref(x), "bf16", f"small batch B={B} T={T}")


@pytest.mark.parametrize("route", ["split", "persistent"])
def test_balanced_all_sequences_empty_and_clamped_lengths(gpu_lib, route):
    """A batch with no cached token at all (the persistent kernel sees N = 0 items) gives zero
    rows over a NaN-filled output; lengths past what the page-table row addresses are clamped
    to it."""
    print(f"[balanced] all empty / clamped {route}", flush=True)
    for dtype, hq, hkv in (("bf16", 32, 8), ("f32", 8, 2), ("bf16", 32, 2)):
        if route == "persistent" and hq // hkv > 8:
            continue
        x = _bal_inputs(gpu_lib, route, 3, hq, hkv, 128, [0, 0, 0], dtype, seed=61)
        out = torch.full_like(x.q, float("nan"))
        gpu_lib.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                      scale=x.scale, out=out)
        _sync()
        assert torch.all(out == 0), f"all empty {dtype} {hq}x{hkv}"
    # rows 1 and 2 fill their page-table rows (mp pages), row 0 holds 40 tokens; only rows
    # whose table is full get a length past it
    mp = 4 if route == "split" else 342  # 3 * 8 * 342 = 8208 items > 8192: persistent
    full = mp * 16
    x = _bal_inputs(gpu_lib, route, 3, 32, 8, 128, [40, full, full], "bf16", seed=62)
    assert x.page_table.shape[1] == mp
    ref = _ref(x)
    big = torch.tensor([40, full + 10_000, 2**30], dtype=torch.int32, device=DEV)
    out = gpu_lib.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, big,
                                        scale=x.scale)
    _sync()
    assert_close(out, ref, "bf16", f"balanced clamped lengths {route}")


@pytest.mark.parametrize("B,hq,hkv,mp,route", [
    (4, 32, 8, 32, "split"), (1, 32, 8, 129, "persistent"),       # G = 4: 1,024 / 1,032 items
    (8, 32, 8, 128, "split"), (8, 32, 8, 129, "persistent"),      # G = 4, 4 splits: 8,192 / 8,256
    (8, 32, 16, 128, "split"), (8, 32, 16, 129, "persistent"),    # G = 2: 16,384 / 16,512
    (2, 8, 8, 4096, "split"), (1, 1, 1, 65537, "persistent"),     # G = 1: 65,536 / 65,537
])
def test_balanced_route_limit_parity(gpu_lib, B, hq, hkv, mp, route):
    """Both sides of the small-problem limit of the balanced entry point match the oracle."""
    print(f"[balanced] route limit B={B} {hq}x{hkv} max_pages={mp} {route}", flush=True)
    lens = [(37 * (b + 3)) % (mp * 16) + 1 for b in range(B)]
    x = synth.decode_inputs(B, hq, hkv, 128, 16, lens, "bf16", seed=mp + B, device=DEV,
                            max_pages=mp)
    assert B * hkv * mp in (1024, 1032, 8192, 8256, 16384, 16512, 65536, 65537)
    assert (gpu_lib.balanced_route(B, hq, hkv, 128, mp) == 0) == (route == "persistent")
    assert_close(_run_bal(gpu_lib, x), _ref(x), "bf16", f"route limit {route}")


def test_balanced_long_context_repeats_are_bitwise_identical(gpu_lib):
    """Workload 4 at B = 1 (one sequence of 32,768 tokens: each of its 8 units is cut into
    hundreds of pieces merged in two levels through device-scope counters): 50 calls in a row
    on one workspace give bit-identical outputs (an ordering fault in the merge would show as
    a differing or unwritten row)."""
    print("[balanced] config4 B=1 x50", flush=True)
    x = synth.config4(1, device=DEV)
    assert gpu_lib.balanced_route(1, 32, 8, 128, x.page_table.shape[1]) == 0
    ws = gpu_lib.balanced_workspace(1, 32, 8, 128, DEV)
    first = None
    for i in range(50):
        out = torch.full_like(x.q, float("nan"))
        gpu_lib.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                      scale=x.scale, out=out, workspace=ws)
        _sync()
        if first is None:
            first = out
            assert torch.isfinite(first.float()).all()
        else:
            assert torch.equal(out, first), f"call {i} differs from the first"


def test_balanced_workspace_reused_across_shapes(gpu_lib):
    """One zero-filled workspace serves a run of calls with different head shapes and length
    mixes (units cut into 2 pieces, into hundreds of pieces, empty sequences, the G >= 16 split
    path in between): every result matches the oracle, rows of empty sequences are written as
    zeros over a NaN-filled output, and the leading counters are zero again after every call
    (so a launch replayed with the same epoch also starts from zero)."""
    import gqa_paged_kv_amd as gk
    cases = [
        ("bf16", 32, 8, [37, 300, 16, 0, 1000, 5, 0, 64]),
        ("bf16", 32, 8, [4096]),          # one sequence: each unit cut into many pieces
        ("bf16", 32, 2, [33] * 40),       # G = 16: split path
        ("f32", 8, 2, [0, 257, 1, 3000, 0, 17]),
        ("bf16", 8, 8, [2000, 0, 999]),   # G = 1
        ("bf16", 32, 8, [37, 300, 16, 0, 1000, 5, 0, 64]),
    ]
    size = max(int(gk.load().gqa_decode_balanced_workspace_bytes(len(lens), hq, hkv, 128))
               for (_, hq, hkv, lens) in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    for i, (dtype, hq, hkv, lens) in enumerate(cases):
        print(f"[balanced] workspace reuse {i} {dtype} {hq}x{hkv} B={len(lens)}", flush=True)
        x = synth.decode_inputs(len(lens), hq, hkv, 128, 16, lens, dtype, seed=500 + i,
                                device=DEV)
        out = torch.full_like(x.q, float("nan"))
        gpu_lib.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                      scale=x.scale, out=out, workspace=ws)
        _sync()
        assert_close(out, _ref(x), dtype, f"workspace reuse case {i}")
        for b, t in enumerate(lens):
            if t == 0:
                assert torch.all(out[b] == 0), f"case {i}: empty sequence {b} not zeroed"
        assert torch.all(ws[:gk.BALANCED_WS_RESERVED] == 0), f"case {i}: counters left non-zero"


# ---------------------------------------------------------------- scale sign and magnitude

@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.7])
@pytest.mark.parametrize("path", ["split1", "split3", "balanced_split", "balanced_persistent",
                                  "balanced_g16"])
def test_decode_scale_sign_and_magnitude(gpu_lib, scale, path):
    """The kernels take the row max of raw q.k and apply the scale in the exponent; a negative
    scale (the max becomes the min), a zero scale (uniform weights; dead slots must still get
    weight 0) and a large one must all match the oracle. Ragged lengths leave dead slots."""
    print(f"[decode] scale {scale} {path}", flush=True)
    hq, hkv = (32, 2) if path == "balanced_g16" else (8, 2)
    if path.startswith("balanced"):
        route = "persistent" if path == "balanced_persistent" else "split"
        x = _bal_inputs(gpu_lib, route, 3, hq, hkv, 128, [37, 200, 5], "bf16", seed=91)
    else:
        x = synth.decode_inputs(3, hq, hkv, 128, 16, [37, 200, 5], "bf16", seed=91, device=DEV)
    x.scale = scale
    if path.startswith("split"):
        out = _run(gpu_lib, x, ns=int(path[-1]))
    else:
        out = _run_bal(gpu_lib, x)
    assert_close(out, _ref(x), "bf16", f"decode scale={scale} {path}")


# ---------------------------------------------------------------- shared-prefix pages

def _shared_prefix_inputs(dtype, hq, hkv, prefix, tails, seed):
    """Beams / sequences that share the physical pages of a common prefix: sequence b's page
    table starts with the same ceil(prefix/P)... pages (the prefix must end on a page
    boundary to be shareable), then private pages for its own tail."""
    P = 16
    assert prefix % P == 0
    lens = [prefix + t for t in tails]
    x = synth.decode_inputs(len(tails), hq, hkv, 128, P, lens, dtype, seed=seed, poison=False)
    pt = x.page_table.clone()
    npre = prefix // P
    pt[:, :npre] = pt[0, :npre]  # every sequence reads sequence 0's prefix pages
    x.page_table = pt
    return x


@pytest.mark.parametrize("path", ["split1", "split4", "balanced"])
@pytest.mark.parametrize("dtype,hq,hkv", [("bf16", 32, 8), ("f32", 8, 2), ("bf16", 32, 2)])
def test_shared_prefix_pages(gpu_lib, path, dtype, hq, hkv):
    """Page-table aliasing: 5 sequences share a 160-token prefix and differ after it. The
    kernels only read the pool, so aliased pages must give exactly the oracle's result."""
    print(f"[decode] shared prefix {path} {dtype} {hq}x{hkv}", flush=True)
    x = _shared_prefix_inputs(dtype, hq, hkv, 160, [0, 1, 15, 16, 300], seed=71).to(DEV)
    out = _run(gpu_lib, x, ns=int(path[-1])) if path.startswith("split") else _run_bal(gpu_lib, x)
    assert_close(out, _ref(x), dtype, f"shared prefix {path}")
    # sequence 0 holds exactly the prefix: every other sequence's prefix part is its prefix
    assert int(x.context_lens[0]) == 160


def test_shared_prefix_identical_sequences_give_identical_rows(gpu_lib):
    """Two sequences with the same page-table row, length and query give bit-identical rows on
    the split path (its split boundaries are relative to each sequence). The balanced
    partition cuts each sequence where the global share boundaries fall, so its two rows are
    summed in different pieces: both must match the oracle."""
    print("[decode] shared prefix identical", flush=True)
    x = synth.decode_inputs(3, 32, 8, 128, 16, [500, 777, 500], "bf16", seed=72, poison=False)
    x.page_table[2] = x.page_table[0]
    x.q[2] = x.q[0]
    x = x.to(DEV)
    ref = _ref(x)
    for ns in (1, 4):
        out = _run(gpu_lib, x, ns)
        assert torch.equal(out[0], out[2]), f"split path ns={ns}"
        assert_close(out, ref, "bf16", f"identical beams ns={ns}")
    out = _run_bal(gpu_lib, x)
    assert_close(out, ref, "bf16", "identical beams (balanced)")
