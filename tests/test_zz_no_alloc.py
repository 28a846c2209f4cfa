"""The allocation-free balanced decode (gqa_decode_paged_balanced_noalloc, the library's
static device scratch) against the workspace entry point (gqa_decode_paged_balanced): two
calls in a row on one device, the second smaller, on each route of the balanced decode."""

import pytest
import torch

import synth
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(g, x):
    want = g.decode_paged_balanced(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                   scale=x.scale)
    got = torch.full_like(x.q, float("nan"))
    g.decode_paged_balanced_noalloc(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                    got, scale=x.scale)
    torch.cuda.synchronize()
    return got, want


def _check(g, x, what):
    got, want = _both(g, x)
    dtype = "f32" if x.q.dtype == torch.float32 else "bf16"
    assert_close(got, want, dtype, what)
    assert torch.equal(got, want), f"{what}: not bit-identical to the workspace entry point"


CASES = {
    # route: (first call, second smaller call) as decode_inputs arguments
    "persistent": (dict(B=64, Hq=32, Hkv=8, lens=(512, 4096), dtype="bf16", seed=2000),
                   dict(B=5, Hq=32, Hkv=8, lens=[700, 0, 33, 1500, 16], dtype="bf16", seed=7,
                        max_pages=100)),
    "split_g32": (dict(B=64, Hq=32, Hkv=1, lens=1024, dtype="bf16", seed=31),
                  dict(B=3, Hq=32, Hkv=1, lens=[100, 513, 7], dtype="bf16", seed=32)),
    "split_small": (dict(B=4, Hq=8, Hkv=2, lens=[300, 511, 64, 1], dtype="f32", seed=41,
                         max_pages=64),
                    dict(B=2, Hq=8, Hkv=2, lens=[40, 200], dtype="f32", seed=42)),
}


@pytest.mark.parametrize("route", list(CASES))
def test_noalloc_matches_workspace_entry_two_calls(gpu_lib, route):
    for i, kw in enumerate(CASES[route]):
        kw = dict(kw)
        B, hq, hkv = kw.pop("B"), kw.pop("Hq"), kw.pop("Hkv")
        lens, dtype, seed = kw.pop("lens"), kw.pop("dtype"), kw.pop("seed")
        print(f"[noalloc] {route} call {i + 1}: B={B} {hq}x{hkv}", flush=True)
        x = synth.decode_inputs(B, hq, hkv, 128, 16, lens, dtype, seed=seed, device=DEV, **kw)
        r = gpu_lib.balanced_route(B, hq, hkv, 128, x.page_table.shape[1],
                                   gpu_lib.NOALLOC_SCRATCH_BYTES)
        assert (r == 0) == (route == "persistent"), f"route {r}"
        _check(gpu_lib, x, f"noalloc {route} call {i + 1}")
