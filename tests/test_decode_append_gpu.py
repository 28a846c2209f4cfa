"""GPU parity of one decode step with its own token appended (gqa_decode_append)."""

import pytest
import torch

import oracle
import synth
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"
P = 16


def _inputs(dtype, hq, hkv, D, lens, seed):
    """Pool and page table sized for lens + 1 tokens; context_lens = lens (tokens before the
    step); the new tokens' slots hold NaN before the call; k_new / v_new drawn after."""
    x = synth.decode_inputs(len(lens), hq, hkv, D, P, [t + 1 for t in lens], dtype, seed=seed)
    x.context_lens = torch.tensor(lens, dtype=torch.int32)
    for b, t in enumerate(lens):
        page = int(x.page_table[b, t // P])
        x.k_cache[page, :, t % P, :] = float("nan")
        x.v_cache[page, :, t % P, :] = float("nan")
    gen = torch.Generator().manual_seed(seed + 1)
    kn = torch.randn((len(lens), hkv, D), generator=gen).to(x.q.dtype)
    vn = torch.randn((len(lens), hkv, D), generator=gen).to(x.q.dtype)
    return x, kn, vn


def _reference(x, kn, vn):
    """Oracle: append at position T_b (append_paged_at with one new row), then decode over
    T_b + 1 tokens."""
    ones = torch.ones_like(x.context_lens)
    kc = oracle.append_paged_at(x.k_cache, kn[:, None], x.page_table, x.context_lens, ones, P)
    vc = oracle.append_paged_at(x.v_cache, vn[:, None], x.page_table, x.context_lens, ones, P)
    out = oracle.decode_paged(x.q, kc, vc, x.page_table, x.context_lens + 1, x.scale)
    return out, kc, vc


def _step(g, x, kn, vn):
    out = g.decode_append(x.q, kn, vn, x.k_cache, x.v_cache, x.page_table, x.context_lens,
                          scale=x.scale)
    torch.cuda.synchronize()
    return out


CASES = [
    # dtype, Hq, Hkv, D, lens
    ("bf16", 32, 8, 128, [0, 1, 15, 16, 17, 100]),
    ("bf16", 8, 8, 128, [31, 32, 33]),
    ("bf16", 16, 8, 64, [5, 250]),
    ("bf16", 32, 4, 128, [1000, 7]),
    ("f32", 8, 2, 128, [16, 47]),
    ("f32", 8, 1, 64, [63, 64, 0]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}x{c[2]}-D{c[3]}")
def test_decode_append_small(gpu_lib, case):
    dtype, hq, hkv, D, lens = case
    print(f"[append] {case}", flush=True)
    x, kn, vn = _inputs(dtype, hq, hkv, D, lens, seed=hq + D + len(lens))
    ref, kc, vc = _reference(x, kn, vn)
    xd = x.to(DEV)
    out = _step(gpu_lib, xd, kn.to(DEV), vn.to(DEV))
    assert_close(out, ref, dtype, f"append {case}")
    view = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(xd.k_cache.cpu().view(view), kc.view(view))
    assert torch.equal(xd.v_cache.cpu().view(view), vc.view(view))


def test_decode_append_three_steps_workload2_shape(gpu_lib):
    """Three consecutive steps at the workload-2 head shape (lens advanced on the host): the
    outputs of every step and the final pool against the oracle run step by step."""
    print("[append] three steps", flush=True)
    lens = [511, 512, 1023, 2000, 17, 4095, 3000, 64]
    B = len(lens)
    x = synth.decode_inputs(B, 32, 8, 128, P, [t + 3 for t in lens], "bf16", seed=77)
    x.context_lens = torch.tensor(lens, dtype=torch.int32)
    gen = torch.Generator().manual_seed(78)
    xd = x.to(DEV)
    kc, vc = x.k_cache.clone(), x.v_cache.clone()
    for step in range(3):
        kn = torch.randn((B, 8, 128), generator=gen).to(torch.bfloat16)
        vn = torch.randn((B, 8, 128), generator=gen).to(torch.bfloat16)
        q = torch.randn((B, 32, 128), generator=gen).to(torch.bfloat16)
        xd.q = q.to(DEV)
        out = _step(gpu_lib, xd, kn.to(DEV), vn.to(DEV))
        ones = torch.ones(B, dtype=torch.int32)
        cl = x.context_lens + step
        kc = oracle.append_paged_at(kc, kn[:, None], x.page_table, cl, ones, P)
        vc = oracle.append_paged_at(vc, vn[:, None], x.page_table, cl, ones, P)
        ref = oracle.decode_paged(q, kc, vc, x.page_table, cl + 1, x.scale)
        assert_close(out, ref, "bf16", f"append step {step}")
        xd.context_lens += 1
    assert torch.equal(xd.k_cache.cpu().view(torch.int16), kc.view(torch.int16))


def test_decode_append_with_shared_prefix(gpu_lib):
    """Beams share the prefix pages and append into private pages."""
    print("[append] shared prefix", flush=True)
    lens = [160, 170, 200]
    x, kn, vn = _inputs("bf16", 32, 8, 128, lens, seed=79)
    x.page_table[1:, :10] = x.page_table[0, :10]  # 160 tokens = 10 shared pages
    # sequence 0 appends at 160: its page 10 is private; so are the others' pages >= 10
    ref, kc, vc = _reference(x, kn, vn)
    xd = x.to(DEV)
    out = _step(gpu_lib, xd, kn.to(DEV), vn.to(DEV))
    assert_close(out, ref, "bf16", "append shared prefix")
    assert torch.equal(xd.k_cache.cpu().view(torch.int16), kc.view(torch.int16))


def test_decode_append_at_capacity_and_clamped(gpu_lib):
    """The page-table row addresses 48 tokens (3 pages): a sequence holding 47 tokens appends
    into the very last slot; a length past the row is clamped so that the append still lands
    in the last slot and the step attends all 48 tokens."""
    print("[append] capacity / clamp", flush=True)
    x, kn, vn = _inputs("bf16", 32, 8, 128, [47, 47], seed=77)
    assert x.page_table.shape[1] == 3
    ref, kc, vc = _reference(x, kn, vn)
    xd = x.to(DEV)
    xd.context_lens = torch.tensor([47, 5000], dtype=torch.int32, device=DEV)
    out = _step(gpu_lib, xd, kn.to(DEV), vn.to(DEV))
    assert_close(out, ref, "bf16", "append at capacity / clamped")
    assert torch.equal(xd.k_cache.cpu().view(torch.int16), kc.view(torch.int16))
    assert torch.equal(xd.v_cache.cpu().view(torch.int16), vc.view(torch.int16))
