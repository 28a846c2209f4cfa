"""GPU parity of paged GQA decode over an 8-bit (E4M3 / E5M2) KV pool (gqa_decode_paged_fp8)."""

import pytest
import torch

import oracle
import synth
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _ref(x):
    c = x.to("cpu")
    return oracle.decode_paged_fp8(c.q, c.k_cache, c.v_cache, c.k_scale, c.v_scale,
                                   c.page_table, c.context_lens, c.scale, c.fmt)


def _run(g, x):
    out = g.decode_paged_fp8(x.q, x.k_cache, x.v_cache, x.k_scale, x.v_scale, x.page_table,
                             x.context_lens, fmt=x.fmt, scale=x.scale)
    torch.cuda.synchronize()
    return out


SMALL = [
    # Hq, Hkv, lens
    (4, 4, [1, 16, 17]),
    (8, 4, [0, 33, 200]),
    (16, 4, [5, 64, 1000, 2]),
    (32, 4, [300, 301]),
    (8, 1, [47]),
]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"{c[0]}x{c[1]}-{len(c[2])}seq")
def test_fp8_decode_small_shapes(gpu_lib, fmt, case):
    hq, hkv, lens = case
    print(f"[fp8] {fmt} {case}", flush=True)
    x = synth.fp8_decode_inputs(len(lens), hq, hkv, 128, 16, lens, fmt,
                                seed=hq + 3 * hkv + len(lens), device=DEV)
    assert_close(_run(gpu_lib, x), _ref(x), "bf16", f"fp8 {fmt} {case}")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_workload2(gpu_lib, fmt):
    """Workload 2 (B=64, Hq=32, Hkv=8, T ~ U[512, 4096], permuted pages, NaN in dead slots)
    with an 8-bit pool: every output row against the oracle, and bit-identical reruns."""
    print(f"[fp8] workload 2 {fmt}", flush=True)
    x = synth.config2_fp8(fmt, device=DEV)
    a = _run(gpu_lib, x)
    assert_close(a, _ref(x), "bf16", f"fp8 workload 2 {fmt}")
    assert torch.equal(a, _run(gpu_lib, x))


def test_fp8_decode_scales_fold_exactly(gpu_lib):
    """Doubling k_scale doubles every score (same as doubling the softmax scale) and
    doubling v_scale doubles the output: both against the oracle."""
    print("[fp8] scales", flush=True)
    x = synth.fp8_decode_inputs(2, 8, 2, 128, 16, [90, 31], "e4m3", seed=8, device=DEV)
    x.k_scale *= 2.0
    x.v_scale *= 0.5
    assert_close(_run(gpu_lib, x), _ref(x), "bf16", "fp8 rescaled")


def test_fp8_decode_all_empty_and_clamped(gpu_lib):
    """No cached token in the whole batch: zero rows over a NaN-filled output. Lengths past
    what the page table addresses are clamped to it."""
    print("[fp8] all empty / clamped", flush=True)
    x = synth.fp8_decode_inputs(2, 32, 8, 128, 16, [0, 0], "e4m3", seed=63, device=DEV)
    out = torch.full_like(x.q, float("nan"))
    gpu_lib.decode_paged_fp8(x.q, x.k_cache, x.v_cache, x.k_scale, x.v_scale, x.page_table,
                             x.context_lens, fmt=x.fmt, scale=x.scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 0)
    y = synth.fp8_decode_inputs(2, 32, 8, 128, 16, [30, 48], "e5m2", seed=64, device=DEV)
    c = y.to("cpu")
    big = torch.tensor([30, 1_000_000], dtype=torch.int32, device=DEV)  # 3 pages per row
    got = gpu_lib.decode_paged_fp8(y.q, y.k_cache, y.v_cache, y.k_scale, y.v_scale,
                                   y.page_table, big, fmt=y.fmt, scale=y.scale)
    torch.cuda.synchronize()
    want = oracle.decode_paged_fp8(c.q, c.k_cache, c.v_cache, c.k_scale, c.v_scale,
                                   c.page_table, torch.tensor([30, 48], dtype=torch.int32),
                                   c.scale, c.fmt)
    assert_close(got, want, "bf16", "fp8 clamped")


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_long_context_multilevel_merge(gpu_lib, fmt):
    """A 32,768-token sequence next to a 100-token one (Hq=32, Hkv=8): each of the long
    sequence's units spans hundreds of wave shares, so its pieces are merged in groups and
    then the group partials are merged (the matrix-core PV's blocks pass through the same
    per-lane layout first). Every output row against the oracle, and a bit-identical rerun."""
    print(f"[fp8] long context {fmt}", flush=True)
    x = synth.fp8_decode_inputs(2, 32, 8, 128, 16, [32768, 100], fmt, seed=4096, device=DEV)
    a = _run(gpu_lib, x)
    assert_close(a, _ref(x), "bf16", f"fp8 long context {fmt}")
    assert torch.equal(a, _run(gpu_lib, x))
