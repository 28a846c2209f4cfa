"""The debug build of the library (libgqa_debug.so: entry points compiled with GQA_DEBUG)
checks every page id a call would touch against the pool on the host and refuses the call,
with nothing enqueued, when one lies outside [0, num_pages)."""

import ctypes
import os

import pytest
import torch

import gqa_paged_kv_amd as g
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def dbg(gpu_lib):
    path = os.path.join(g.HERE, "libgqa_debug.so")
    if not os.path.exists(path):
        pytest.fail("libgqa_debug.so is missing: build it with `python -m gqa_paged_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (ret, args) in g.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = ret, args
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _decode(lib, x, num_pages, out):
    B, Hq, D = x.q.shape
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gqa_decode_paged(_p(x.q), _p(x.k_cache), _p(x.v_cache), _p(x.page_table),
                                _p(x.context_lens), _p(out), None, None, B, Hq,
                                x.k_cache.shape[1], D, 16, x.page_table.shape[1], num_pages, 1,
                                x.scale, g.BF16, s)


def test_debug_build_rejects_page_ids_outside_the_pool(dbg, gpu_lib):
    print("[debug lib] page ids", flush=True)
    x = synth.decode_inputs(3, 8, 2, 128, 16, [40, 300, 17], "bf16", seed=3, device=DEV)
    n_alloc = x.k_cache.shape[0]
    out = torch.full_like(x.q, float("nan"))
    # declared pool = every allocated page: accepted, same result as the release build
    assert _decode(dbg, x, n_alloc, out) == g.OK
    torch.cuda.synchronize()
    want = gpu_lib.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                                scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    # a live entry names the last allocated page while the declared pool ends before it: the
    # check refuses the call (the page would still be inside the allocation, had it run)
    pt = x.page_table.clone()
    pt[1, 5] = n_alloc - 1
    y = synth.DecodeInputs(x.q, x.k_cache, x.v_cache, pt, x.context_lens, x.scale)
    out2 = torch.full_like(x.q, float("nan"))
    assert _decode(dbg, y, n_alloc - 1, out2) == g.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.isnan(out2.float()).all(), "nothing may be enqueued on a refused call"
    # an entry past the last live page is never read, so any value there is accepted
    pt2 = x.page_table.clone()
    pt2[2, 2:] = 10**6  # sequence 2 holds 17 tokens: pages 0 and 1
    z = synth.DecodeInputs(x.q, x.k_cache, x.v_cache, pt2, x.context_lens, x.scale)
    assert _decode(dbg, z, n_alloc, out) == g.OK
    torch.cuda.synchronize()
    assert torch.equal(out, want)
