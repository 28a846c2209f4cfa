"""Pins for the float64 oracle (CPU only).

The oracle is checked against things other than itself: a pure-Python brute
force, closed forms (identical keys / zero query give the mean of V; one
token gives V[0] exactly), torch's float64 SDPA with ``enable_gqa`` (a library
routine whose GQA mapping is the contiguous one), invariants (page
permutation, repeat_kv expansion, split count, key shift, convex hull) and
the KV-size ratio printed on the GQA/TensorRT page. A few tests plant a
mistake in the oracle and check that a pin catches it.
"""

import json
import math
import os
import random

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as oa
from oracle import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tol_close(a, b, rel=1e-13):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(1.0, float(np.abs(b).max()) if b.size else 1.0)
    return float(np.abs(a - b).max()) <= rel * scale if a.size else True


def _small_decode(seed, B, hq, hkv, D, P, lens, dtype="f32", **kw):
    return synth.decode_inputs(B, hq, hkv, D, P, lens, dtype, seed=seed, pad_pages=3, **kw)


def _contiguous_to_paged(kc, vc, P, seed, pad=2):
    """Test-side scatter of contiguous K/V [B][Hkv][T][D] into a permuted pool."""
    B, hkv, T, D = kc.shape
    npg = (T + P - 1) // P
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * npg + pad, generator=g)[: B * npg]
    pool_k = torch.full((B * npg + pad, hkv, P, D), float("nan"), dtype=kc.dtype)
    pool_v = pool_k.clone()
    pt = torch.full((B, npg + 1), -1, dtype=torch.int32)
    for b in range(B):
        for i in range(npg):
            phys = int(perm[b * npg + i])
            pt[b, i] = phys
            for s in range(P):
                t = i * P + s
                if t < T:
                    pool_k[phys, :, s, :] = kc[b, :, t, :]
                    pool_v[phys, :, s, :] = vc[b, :, t, :]
    return pool_k, pool_v, pt


# ---------------------------------------------------------------- brute force

DECODE_CASES = [
    # B, Hq, Hkv, D, P, lens
    (1, 1, 1, 1, 1, [5]),
    (2, 2, 1, 3, 4, [7, 1]),
    (2, 4, 2, 8, 4, [23, 16]),
    (1, 8, 2, 5, 8, [17]),
    (2, 4, 4, 4, 8, [9, 0]),
    (2, 8, 1, 6, 1, [3, 11]),
]


@pytest.mark.parametrize("case", DECODE_CASES)
def test_decode_matches_brute_force(case):
    B, hq, hkv, D, P, lens = case
    x = _small_decode(11 + len(lens) + D, B, hq, hkv, D, P, lens)
    got = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    ref = brute.decode(x.q.double().tolist(), x.k_cache.double().tolist(),
                       x.v_cache.double().tolist(), x.page_table.tolist(),
                       x.context_lens.tolist(), x.scale)
    assert _tol_close(got, ref)
    assert np.isfinite(got).all()


PREFILL_CASES = [(1, 1, 1, 1, 2), (2, 5, 2, 1, 3), (1, 9, 4, 2, 8), (2, 6, 8, 2, 4), (1, 7, 4, 4, 5)]


@pytest.mark.parametrize("case", PREFILL_CASES)
def test_prefill_matches_brute_force(case):
    B, S, hq, hkv, D = case
    x = synth.prefill_inputs(B, S, hq, hkv, D, 4, seed=21 + S, dtype="f32")
    got = oracle.prefill_causal(x.q, x.k, x.v, x.scale)
    ref = brute.prefill(x.q.double().tolist(), x.k.double().tolist(), x.v.double().tolist(), x.scale)
    assert _tol_close(got, ref)


# ------------------------------------------------------------- closed forms

def test_identical_keys_give_mean_of_values():
    x = _small_decode(5, 2, 8, 2, 16, 4, [13, 30])
    k0 = torch.randn(16, generator=torch.Generator().manual_seed(3))
    kc = x.k_cache.clone()
    kc[:] = k0  # every key row identical (pads too; they are never read)
    got = oracle.decode_paged(x.q, kc, x.v_cache, x.page_table, x.context_lens, x.scale)
    for b in range(2):
        T = int(x.context_lens[b])
        for h in range(8):
            g = h // 4
            vals = [x.v_cache[int(x.page_table[b, t // 4]), g, t % 4].double() for t in range(T)]
            mean = torch.stack(vals).mean(0).numpy()
            assert np.abs(got[b, h] - mean).max() <= 1e-13


def test_zero_query_gives_mean_of_values():
    x = _small_decode(6, 1, 4, 1, 8, 8, [21])
    q0 = torch.zeros_like(x.q)
    got = oracle.decode_paged(q0, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    vals = [x.v_cache[int(x.page_table[0, t // 8]), 0, t % 8].double() for t in range(21)]
    mean = torch.stack(vals).mean(0).numpy()
    assert np.abs(got[0] - mean[None, :]).max() <= 1e-13


def test_single_token_is_exact_value_row():
    x = _small_decode(7, 2, 4, 2, 8, 4, [1, 1])
    got = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    for b in range(2):
        for h in range(4):
            v0 = x.v_cache[int(x.page_table[b, 0]), h // 2, 0].double().numpy()
            assert np.array_equal(got[b, h], v0)


def test_prefill_identical_keys_give_running_mean():
    x = synth.prefill_inputs(1, 12, 4, 2, 8, 4, seed=9, dtype="f32")
    k = x.k.clone()
    k[:] = 0.5
    got = oracle.prefill_causal(x.q, k, x.v, x.scale)
    v = x.v.double().numpy()
    for i in range(12):
        for h in range(4):
            mean = v[0, : i + 1, h // 2, :].mean(0)
            assert np.abs(got[0, i, h] - mean).max() <= 1e-13
    # row 0 sees only key 0: exactly V[0]
    for h in range(4):
        assert np.array_equal(got[0, 0, h], v[0, 0, h // 2])


# ------------------------------------------------------ library routine (SDPA)

@pytest.mark.parametrize("hq,hkv", [(8, 2), (8, 8), (4, 1), (32, 8)])
def test_decode_matches_torch_sdpa_gqa(hq, hkv):
    B, T, D, P = 2, 37, 16, 8
    g = torch.Generator().manual_seed(hq * 100 + hkv)
    q = torch.randn(B, hq, D, generator=g, dtype=torch.float64)
    kc = torch.randn(B, hkv, T, D, generator=g, dtype=torch.float64)
    vc = torch.randn(B, hkv, T, D, generator=g, dtype=torch.float64)
    pk, pv, pt = _contiguous_to_paged(kc, vc, P, seed=hq + hkv)
    lens = torch.full((B,), T, dtype=torch.int32)
    scale = 1 / math.sqrt(D)
    got = oracle.decode_paged(q, pk, pv, pt, lens, scale)
    ref = F.scaled_dot_product_attention(q[:, :, None, :], kc, vc, scale=scale,
                                         enable_gqa=True)[:, :, 0, :]
    assert np.abs(got - ref.numpy()).max() <= 1e-12


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 1)])
def test_prefill_matches_torch_sdpa_causal_gqa(hq, hkv):
    B, S, D = 2, 29, 8
    g = torch.Generator().manual_seed(7 * hq + hkv)
    q = torch.randn(B, S, hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(B, S, hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(B, S, hkv, D, generator=g, dtype=torch.float64)
    scale = 1 / math.sqrt(D)
    got = oracle.prefill_causal(q, k, v, scale)
    ref = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2).contiguous(),
                                         v.transpose(1, 2).contiguous(), scale=scale,
                                         is_causal=True, enable_gqa=True).transpose(1, 2)
    assert np.abs(got - ref.numpy()).max() <= 1e-12


# ---------------------------------------------------------------- invariants

def test_repeat_kv_expansion_is_identical_mha():
    x = _small_decode(8, 2, 8, 2, 8, 4, [19, 6])
    gqa = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    ke = x.k_cache.repeat_interleave(4, dim=1)
    ve = x.v_cache.repeat_interleave(4, dim=1)
    mha = oracle.decode_paged(x.q, ke, ve, x.page_table, x.context_lens, x.scale)
    assert np.array_equal(gqa, mha)


def test_page_permutation_leaves_output_bit_identical():
    x = _small_decode(9, 3, 8, 2, 8, 4, [17, 4, 30])
    base = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    n = x.k_cache.shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1))  # old -> new id
    k2 = torch.empty_like(x.k_cache)
    v2 = torch.empty_like(x.v_cache)
    k2[perm] = x.k_cache
    v2[perm] = x.v_cache
    pt2 = x.page_table.clone()
    live = pt2 >= 0
    pt2[live] = perm[pt2[live].long()].to(torch.int32)
    moved = oracle.decode_paged(x.q, k2, v2, pt2, x.context_lens, x.scale)
    assert np.array_equal(base, moved)


@pytest.mark.parametrize("ns", [1, 2, 3, 4, 8, 16])
def test_split_and_combine_equals_unsplit(ns):
    x = _small_decode(10, 3, 4, 2, 8, 4, [45, 7, 64])
    ref = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    o, lse = oracle.decode_split_partials(x.q, x.k_cache, x.v_cache, x.page_table,
                                          x.context_lens, x.scale, ns)
    assert _tol_close(oracle.combine_splits(o, lse), ref)
    # an empty split is marked -inf with a zero output
    for b, T in enumerate([45, 7, 64]):
        npg = -(-T // 4)
        for s, (lo, hi) in enumerate(oracle.split_page_ranges(npg, ns)):
            if hi <= lo:
                assert np.all(lse[b, :, s] == -np.inf) and np.all(o[b, :, s] == 0)


def test_split_lse_matches_brute_logsumexp():
    x = _small_decode(12, 1, 2, 1, 4, 4, [10])
    o, lse = oracle.decode_split_partials(x.q, x.k_cache, x.v_cache, x.page_table,
                                          x.context_lens, x.scale, 3)
    q = x.q.double().tolist()
    for s, (lo, hi) in enumerate(oracle.split_page_ranges(3, 3)):
        for h in range(2):
            scores = []
            for t in range(lo * 4, min(hi * 4, 10)):
                p = int(x.page_table[0, t // 4])
                k = x.k_cache[p, 0, t % 4].double().tolist()
                scores.append(x.scale * math.fsum(q[0][h][c] * k[c] for c in range(4)))
            m = max(scores)
            expect = m + math.log(math.fsum(math.exp(v - m) for v in scores))
            assert abs(lse[0, h, s] - expect) <= 1e-13 * max(1.0, abs(expect))


def test_split_page_ranges_cover_exactly():
    for n in range(0, 40):
        for ns in (1, 2, 3, 4, 8, 16):
            r = oracle.split_page_ranges(n, ns)
            assert len(r) == ns
            covered = [p for lo, hi in r for p in range(lo, hi)]
            assert covered == list(range(n))


def test_combine_special_cases():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((4, 5, 3))
    lse = np.full((4, 5), -np.inf)
    out = oracle.combine_splits(o, lse)
    assert np.all(out == 0)  # all splits empty -> zero
    lse[1, 2] = 0.3  # one live split -> that split's output exactly
    out = oracle.combine_splits(o, lse)
    assert np.array_equal(out[1], o[1, 2])
    lse[2, :] = 1.25  # equal weights -> plain mean
    out = oracle.combine_splits(o, lse)
    assert np.abs(out[2] - o[2].mean(0)).max() <= 1e-15
    lse[3] = rng.standard_normal(5)  # a common shift of all lse changes nothing
    a = oracle.combine_splits(o[3:4], lse[3:4])
    b = oracle.combine_splits(o[3:4], lse[3:4] + 40.0)
    assert np.abs(a - b).max() <= 1e-14


def test_convex_hull_and_key_shift():
    x = _small_decode(13, 2, 4, 2, 8, 4, [33, 12])
    out = oracle.decode_paged(x.q, x.k_cache, x.v_cache, x.page_table, x.context_lens, x.scale)
    shifted = x.k_cache.double()  # shift in float64 so the inputs stay exact
    u = torch.randn(8, generator=torch.Generator().manual_seed(4), dtype=torch.float64)
    shifted += u  # every key of every head moves by the same vector
    out2 = oracle.decode_paged(x.q, shifted, x.v_cache, x.page_table, x.context_lens, x.scale)
    assert np.abs(out - out2).max() <= 1e-12
    for b, T in enumerate([33, 12]):
        for h in range(4):
            vals = np.stack([x.v_cache[int(x.page_table[b, t // 4]), h // 2, t % 4].double().numpy()
                             for t in range(T)])
            assert np.all(out[b, h] >= vals.min(0) - 1e-14)
            assert np.all(out[b, h] <= vals.max(0) + 1e-14)


def test_gather_identity_and_permuted():
    kc = torch.randn(2, 3, 21, 4, dtype=torch.float64)
    vc = torch.randn(2, 3, 21, 4, dtype=torch.float64)
    pk, pv, pt = _contiguous_to_paged(kc, vc, 8, seed=3)
    lens = torch.tensor([21, 9], dtype=torch.int32)
    got = oracle.gather_paged(pk, pt, lens, 8)
    assert torch.equal(got[0], kc[0].transpose(0, 1))
    assert torch.equal(got[1], kc[1, :, :9].transpose(0, 1))


def test_append_round_trip_and_untouched_pages():
    x = synth.prefill_inputs(2, 37, 4, 2, 8, 8, seed=4, dtype="bf16")
    kc = oracle.append_paged(x.k_cache, x.k, x.page_table, 8)
    back = oracle.gather_paged(kc, x.page_table, torch.tensor([37, 37]), 8)
    for b in range(2):
        assert torch.equal(back[b], x.k[b])
    used = set(int(p) for p in x.page_table.flatten())
    for p in range(kc.shape[0]):
        if p not in used:
            assert torch.isnan(kc[p].float()).all()


def test_kv_bytes_absolute():
    """kv_bytes counts every cached K and V element once: workload 1's cache (2 sequences of
    256 tokens, 2 KV heads, D = 64, fp32) is 2 * 512 * 2 * 64 * 4 = 524,288 bytes, and for any
    shape it equals the byte size of a dense K tensor plus a dense V tensor [T][Hkv][D] of that
    dtype."""
    assert oracle.kv_bytes(2 * 256, 2, 64, 4) == 524_288
    for T, hkv, d, dt in ((1, 1, 1, torch.bfloat16), (141_394, 8, 128, torch.bfloat16),
                          (37, 3, 64, torch.float32), (1000, 32, 128, torch.uint8)):
        k = torch.empty(T, hkv, d, dtype=dt)
        v = torch.empty(T, hkv, d, dtype=dt)
        dense = k.numel() * k.element_size() + v.numel() * v.element_size()
        assert oracle.kv_bytes(T, hkv, d, k.element_size()) == dense


def test_kv_size_ratio_golden():
    with open(os.path.join(GOLDEN, "kv_cache_ratio.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        mha = oracle.kv_bytes(case["tokens"], case["query_heads"], 128, 2)
        gqa = oracle.kv_bytes(case["tokens"], case["kv_heads"], 128, 2)
        assert gqa / mha == pytest.approx(1 - case["reduction"], abs=0)


# ------------------------------------------------ planted mistakes are caught

def _sdpa_decode_error():
    B, T, D, P, hq, hkv = 1, 20, 8, 4, 8, 2
    g = torch.Generator().manual_seed(99)
    q = torch.randn(B, hq, D, generator=g, dtype=torch.float64)
    kc = torch.randn(B, hkv, T, D, generator=g, dtype=torch.float64)
    vc = torch.randn(B, hkv, T, D, generator=g, dtype=torch.float64)
    pk, pv, pt = _contiguous_to_paged(kc, vc, P, seed=5)
    got = oa.decode_paged(q, pk, pv, pt, torch.tensor([T]), 1 / math.sqrt(D))
    ref = F.scaled_dot_product_attention(q[:, :, None, :], kc, vc, enable_gqa=True)[:, :, 0, :]
    return np.abs(got - ref.numpy()).max()


def test_planted_interleaved_head_mapping_is_caught(monkeypatch):
    assert _sdpa_decode_error() <= 1e-12
    monkeypatch.setattr(oa, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert _sdpa_decode_error() > 1e-3


def test_planted_slot_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "logical_to_physical",
                        lambda row, t, P: (int(row[t // P]), (t + 1) % P))
    x = _small_decode(14, 1, 2, 1, 4, 4, [9])
    x.k_cache[:] = x.k_cache.nan_to_num(0.0)
    x.v_cache[:] = x.v_cache.nan_to_num(0.0)
    got = oa.gather_paged(x.k_cache, x.page_table, x.context_lens, 4)[0]
    want = torch.stack([x.k_cache[int(x.page_table[0, t // 4]), :, t % 4] for t in range(9)])
    assert not torch.equal(got, want)


def test_planted_off_by_one_causal_is_caught(monkeypatch):
    x = synth.prefill_inputs(1, 6, 2, 1, 4, 4, seed=2, dtype="f32")
    ref = brute.prefill(x.q.double().tolist(), x.k.double().tolist(), x.v.double().tolist(), x.scale)
    real_triu = np.triu
    monkeypatch.setattr(oa.np, "triu", lambda m, k=0: real_triu(m, k=k + 1))  # lets j == i+1 in
    got = oa.prefill_causal(x.q, x.k, x.v, x.scale)
    monkeypatch.undo()
    assert not _tol_close(got, ref)


# ------------------------------------------------------------- chunked prefill

CHUNKED = [
    # B, S, Hq, Hkv, D, P, past, new
    (1, 3, 2, 1, 8, 4, [0], [3]),
    (2, 5, 4, 2, 8, 4, [1, 6], [5, 2]),
    (2, 4, 4, 1, 4, 4, [4, 9], [1, 4]),
    (1, 6, 2, 2, 8, 2, [3], [0]),
]


@pytest.mark.parametrize("case", CHUNKED, ids=lambda c: f"B{c[0]}-S{c[1]}-p{c[6]}-n{c[7]}")
def test_chunked_prefill_matches_brute_force(case):
    B, S, hq, hkv, D, P, past, new = case
    x = synth.chunked_inputs(B, S, hq, hkv, D, P, past, new, seed=70 + S, dtype="f32")
    got = oracle.prefill_paged(x.q, x.k_cache, x.v_cache, x.k, x.v, x.page_table, x.past_lens,
                               x.new_lens, x.scale, P)
    ref = brute.prefill_paged(x.q.double().tolist(), x.k_cache.double().tolist(),
                              x.v_cache.double().tolist(), x.k.double().tolist(),
                              x.v.double().tolist(), x.page_table.tolist(), past, new, x.scale)
    for b in range(B):
        if new[b]:
            assert _tol_close(got[b, :new[b]], np.asarray(ref[b]))
        assert np.isnan(got[b, new[b]:]).all()  # rows past the chunk are undefined


def test_chunked_prefill_without_past_is_causal_prefill():
    x = synth.chunked_inputs(2, 9, 4, 2, 16, 4, 0, None, seed=81, dtype="f32")
    got = oracle.prefill_paged(x.q, x.k_cache, x.v_cache, x.k, x.v, x.page_table, x.past_lens,
                               x.new_lens, x.scale, 4)
    assert _tol_close(got, oracle.prefill_causal(x.q, x.k, x.v, x.scale))
    # and its append is the plain append at positions 0..S-1
    a = oracle.append_paged_at(x.k_cache, x.k, x.page_table, x.past_lens, x.new_lens, 4)
    b = oracle.append_paged(x.k_cache, x.k, x.page_table, 4)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_chunked_prefill_single_token_is_decode_after_append():
    past = [0, 5, 16, 23]
    x = synth.chunked_inputs(4, 3, 8, 2, 16, 4, past, 1, seed=82, dtype="f32")
    got = oracle.prefill_paged(x.q, x.k_cache, x.v_cache, x.k, x.v, x.page_table, x.past_lens,
                               x.new_lens, x.scale, 4)
    kc = oracle.append_paged_at(x.k_cache, x.k, x.page_table, x.past_lens, x.new_lens, 4)
    vc = oracle.append_paged_at(x.v_cache, x.v, x.page_table, x.past_lens, x.new_lens, 4)
    dec = oracle.decode_paged(x.q[:, 0], kc, vc, x.page_table, x.past_lens + 1, x.scale)
    assert _tol_close(got[:, 0], dec)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4)])
def test_chunked_prefill_matches_torch_sdpa_bottom_right(hq, hkv):
    """torch's SDPA in float64 with an explicit bottom-right causal mask on the gathered
    context (a library routine independent of the oracle)."""
    B, S, D, P = 2, 6, 16, 4
    past, new = [7, 2], [6, 4]
    x = synth.chunked_inputs(B, S, hq, hkv, D, P, past, new, seed=83 + hq, dtype="f32")
    got = oracle.prefill_paged(x.q, x.k_cache, x.v_cache, x.k, x.v, x.page_table, x.past_lens,
                               x.new_lens, x.scale, P)
    for b in range(B):
        p, n = past[b], new[b]
        t = torch.arange(p)
        pages = x.page_table[b, (t // P)].long()
        K = torch.cat([x.k_cache[pages, :, t % P, :], x.k[b, :n]], 0).double()  # [p+n][Hkv][D]
        V = torch.cat([x.v_cache[pages, :, t % P, :], x.v[b, :n]], 0).double()
        Q = x.q[b, :n].double()
        allowed = torch.arange(p + n)[None, :] <= (p + torch.arange(n))[:, None]
        ref = F.scaled_dot_product_attention(Q.transpose(0, 1), K.transpose(0, 1),
                                             V.transpose(0, 1), attn_mask=allowed,
                                             scale=x.scale, enable_gqa=True)
        assert np.abs(got[b, :n] - ref.transpose(0, 1).numpy()).max() <= 1e-12


def test_chunked_append_leaves_other_slots_untouched():
    x = synth.chunked_inputs(2, 4, 4, 2, 8, 4, [3, 6], [4, 2], seed=84, dtype="f32")
    after = oracle.append_paged_at(x.k_cache, x.k, x.page_table, x.past_lens, x.new_lens, 4)
    changed = ~((after == x.k_cache) | (torch.isnan(after) & torch.isnan(x.k_cache)))
    # exactly the new rows (new_lens tokens x Hkv heads) changed
    assert int(changed.any(-1).sum()) == (4 + 2) * 2
    for b, (p, n) in enumerate([(3, 4), (6, 2)]):
        for i in range(n):
            page, slot = int(x.page_table[b, (p + i) // 4]), (p + i) % 4
            assert torch.equal(after[page, :, slot, :], x.k[b, i])


# ------------------------------------------------------------- 8-bit KV cache

@pytest.mark.parametrize("fmt,tdt", [("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)])
def test_fp8_decoders_match_torch_for_every_byte(fmt, tdt):
    """The bit-level decoders against torch's float8 types (a library routine), all 256 bytes."""
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(tdt).to(torch.float64).numpy()
    got = oracle.fp8.DECODERS[fmt](b.numpy())
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), np.where(~same)


def test_fp8_decoder_special_values():
    d4, d5 = oracle.fp8.decode_e4m3, oracle.fp8.decode_e5m2
    assert d4(np.array([0x7E]))[0] == 448.0 and np.isnan(d4(np.array([0x7F]))[0])
    assert d4(np.array([0x01]))[0] == 2.0 ** -9 and d4(np.array([0xB8]))[0] == -1.0
    assert d5(np.array([0x7B]))[0] == 57344.0 and np.isinf(d5(np.array([0x7C]))[0])
    assert d5(np.array([0x01]))[0] == 2.0 ** -16 and d5(np.array([0x3C]))[0] == 1.0


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_matches_brute_force(fmt):
    """Tiny 8-bit decode against the pure-Python brute force on values dequantized by torch."""
    x = synth.fp8_decode_inputs(2, 4, 2, 16, 4, [7, 10], fmt, seed=55)
    got = oracle.decode_paged_fp8(x.q, x.k_cache, x.v_cache, x.k_scale, x.v_scale,
                                  x.page_table, x.context_lens, x.scale, fmt)
    tdt = synth.FP8_DTYPES[fmt]
    kd = (x.k_cache.view(tdt).double() * x.k_scale).tolist()
    vd = (x.v_cache.view(tdt).double() * x.v_scale).tolist()
    ref = brute.decode(x.q.double().tolist(), kd, vd, x.page_table.tolist(),
                       x.context_lens.tolist(), x.scale)
    assert _tol_close(got, ref)


def test_fp8_quantisation_is_close_to_the_unquantised_decode():
    """Sanity of the synthetic inputs: e4m3 keeps 3 mantissa bits, so the 8-bit decode is
    within a few percent of the fp32 decode it was quantised from."""
    x = synth.fp8_decode_inputs(2, 8, 2, 64, 16, [100, 37], "e4m3", seed=56)
    f = synth.decode_inputs(2, 8, 2, 64, 16, [100, 37], "f32", seed=56)
    a = oracle.decode_paged_fp8(x.q, x.k_cache, x.v_cache, x.k_scale, x.v_scale,
                                x.page_table, x.context_lens, x.scale, "e4m3")
    b = oracle.decode_paged(f.q.to(torch.bfloat16), f.k_cache, f.v_cache, f.page_table,
                            f.context_lens, f.scale)
    assert np.abs(a - b).max() < 0.1
