"""GPU parity of chunked prefill over an existing paged context (gqa_prefill_paged)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import assert_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"
P = 16


def _run_and_check(g, x, what, rows=None):
    """Run on the GPU; compare live rows with the oracle, the cache with the oracle's append
    (bit for bit, NaN pads included) and check that rows past each chunk are untouched."""
    c = x.to("cpu")
    kb, vb = c.k_cache.clone(), c.v_cache.clone()
    sentinel = torch.full_like(x.q, 3.0)
    out = g.prefill_paged(x.q, x.k, x.v, x.k_cache, x.v_cache, x.page_table, x.past_lens,
                          x.new_lens, scale=x.scale, out=sentinel.clone())
    torch.cuda.synchronize()
    out = out.cpu()
    B, S, hq, _ = c.q.shape
    new = [int(n) for n in c.new_lens]
    if rows is None:
        ref = oracle.prefill_paged(c.q, kb, vb, c.k, c.v, c.page_table, c.past_lens, c.new_lens,
                                   c.scale, P)
        got = np.concatenate([to_f64(out[b, :new[b]]) for b in range(B)])
        want = np.concatenate([ref[b, :new[b]] for b in range(B)])
    else:
        ref = oracle.prefill_paged_rows(c.q, kb, vb, c.k, c.v, c.page_table, c.past_lens,
                                        c.new_lens, c.scale, rows, P)
        got = np.concatenate([to_f64(out[b, :new[b], h]) for (b, h) in rows])
        want = np.concatenate([ref[(b, h)] for (b, h) in rows])
    assert_close(got, want, "bf16", what)
    for b in range(B):  # rows past the chunk keep the sentinel
        assert torch.equal(out[b, new[b]:], sentinel[b, new[b]:].cpu()), f"{what}: row >= new"
    want_k = oracle.append_paged_at(kb, c.k, c.page_table, c.past_lens, c.new_lens, P)
    want_v = oracle.append_paged_at(vb, c.v, c.page_table, c.past_lens, c.new_lens, P)
    assert torch.equal(x.k_cache.cpu().view(torch.int16), want_k.view(torch.int16)), what
    assert torch.equal(x.v_cache.cpu().view(torch.int16), want_v.view(torch.int16)), what


SMALL = [
    # B, S, Hq, Hkv, past, new
    (1, 1, 4, 1, [0], [1]),
    (1, 1, 8, 2, [37], [1]),
    (2, 33, 8, 2, [0, 5], [33, 20]),
    (2, 64, 8, 2, [16, 64], [64, 64]),
    (2, 70, 16, 4, [1, 63], [70, 9]),
    (3, 100, 8, 8, [15, 100, 257], [100, 0, 37]),
    (1, 130, 16, 2, [300], [130]),
    (2, 200, 32, 4, [17, 511], [200, 150]),
    (2, 96, 4, 4, [1000, 3], [96, 96]),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-S{}-{}x{}-p{}-n{}".format(*c))
def test_chunked_prefill_small_shapes(gpu_lib, case):
    B, S, hq, hkv, past, new = case
    print(f"[chunked] {case}", flush=True)
    x = synth.chunked_inputs(B, S, hq, hkv, 128, P, past, new, seed=S + 7 * hkv, device=DEV)
    _run_and_check(gpu_lib, x, f"chunked {case}")


def test_chunked_prefill_without_past_matches_causal_prefill(gpu_lib):
    """past = 0, new = S: the same result as gqa_prefill_causal (both against the oracle, and
    the two GPU outputs close to each other)."""
    print("[chunked] past 0", flush=True)
    x = synth.chunked_inputs(2, 300, 8, 2, 128, P, 0, None, seed=9, device=DEV)
    _run_and_check(gpu_lib, x, "chunked past=0")
    y = synth.chunked_inputs(2, 300, 8, 2, 128, P, 0, None, seed=9, device=DEV)
    a = gpu_lib.prefill_paged(y.q, y.k, y.v, y.k_cache, y.v_cache, y.page_table, y.past_lens,
                              y.new_lens, scale=y.scale)
    b = gpu_lib.prefill_causal(y.q, y.k, y.v, y.k_cache.clone(), y.v_cache.clone(),
                               y.page_table, scale=y.scale)
    torch.cuda.synchronize()
    assert_close(a, to_f64(b), "bf16", "chunked vs causal kernel")


def test_chunked_prefill_two_chunks_equal_one_prefill(gpu_lib):
    """Prefill 160 tokens, then a 96-token chunk: the chunk's rows are the last 96 rows of a
    256-token causal prefill (oracle), and the cache holds all 256 tokens."""
    print("[chunked] two chunks", flush=True)
    B, S1, S2, hq, hkv = 2, 160, 96, 8, 2
    full = synth.prefill_inputs(B, S1 + S2, hq, hkv, 128, P, seed=31, device=DEV)
    kc, vc, pt = full.k_cache, full.v_cache, full.page_table
    gpu_lib.prefill_causal(full.q[:, :S1].contiguous(), full.k[:, :S1].contiguous(),
                           full.v[:, :S1].contiguous(), kc, vc, pt, scale=full.scale)
    past = torch.full((B,), S1, dtype=torch.int32, device=DEV)
    new = torch.full((B,), S2, dtype=torch.int32, device=DEV)
    out = gpu_lib.prefill_paged(full.q[:, S1:].contiguous(), full.k[:, S1:].contiguous(),
                                full.v[:, S1:].contiguous(), kc, vc, pt, past, new,
                                scale=full.scale)
    torch.cuda.synchronize()
    c = full.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)[:, S1:]
    assert_close(out, ref, "bf16", "second chunk")
    want = oracle.append_paged(c.k_cache, c.k, c.page_table, P)
    assert torch.equal(kc.cpu().view(torch.int16), want.view(torch.int16))


def test_chunked_prefill_long_context_sampled_heads(gpu_lib):
    """2048 cached tokens + a 512-token chunk per sequence at the benchmark's head shape."""
    print("[chunked] long context", flush=True)
    x = synth.chunked_inputs(2, 512, 32, 8, 128, P, [2048, 1999], [512, 480], seed=4242,
                             device=DEV)
    rows = [(b, h) for b in range(2) for h in (b, 9 + 5 * b, 31 - b)]
    _run_and_check(gpu_lib, x, "chunked long", rows=rows)


def test_chunked_prefill_deterministic(gpu_lib):
    print("[chunked] determinism", flush=True)
    x = synth.chunked_inputs(2, 200, 16, 4, 128, P, [77, 300], [200, 123], seed=5, device=DEV)
    # the second call re-appends the same rows at the same positions; rows past the chunk
    # are untouched, so both outputs start from zeros
    a = gpu_lib.prefill_paged(x.q, x.k, x.v, x.k_cache, x.v_cache, x.page_table, x.past_lens,
                              x.new_lens, scale=x.scale, out=torch.zeros_like(x.q))
    b = gpu_lib.prefill_paged(x.q, x.k, x.v, x.k_cache, x.v_cache, x.page_table, x.past_lens,
                              x.new_lens, scale=x.scale, out=torch.zeros_like(x.q))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_chunked_prefill_items_without_live_rows(gpu_lib):
    """Chunks much shorter than the padded length S: the heaviest q-tiles of a sequence hold
    no live row and are skipped, workgroups of a sequence with an empty chunk do nothing,
    and the others walk several q-tiles; sampled heads against the oracle."""
    print("[chunked] dead items", flush=True)
    x = synth.chunked_inputs(4, 1024, 32, 8, 128, P, [0, 300, 2000, 50], [1024, 500, 64, 0],
                             seed=1717, device=DEV)
    rows = [(0, 3), (0, 30), (1, 9), (1, 17), (2, 0), (2, 31)]
    _run_and_check(gpu_lib, x, "chunked dead items", rows=rows)
