"""GPU parity of causal GQA prefill (bf16 MFMA) and its paged KV append."""

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.helpers import assert_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(g, x):
    out = g.prefill_causal(x.q, x.k, x.v, x.k_cache, x.v_cache, x.page_table, scale=x.scale)
    torch.cuda.synchronize()
    return out


def _check_append(x, k_before, v_before):
    """Cache after append equals the oracle's scatter, bit for bit (NaN pads included)."""
    pt = x.page_table.cpu()
    want_k = oracle.append_paged(k_before, x.k.cpu(), pt, k_before.shape[2])
    want_v = oracle.append_paged(v_before, x.v.cpu(), pt, v_before.shape[2])
    assert torch.equal(x.k_cache.cpu().view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(x.v_cache.cpu().view(torch.int16), want_v.view(torch.int16))


SMALL = [
    # B, S, Hq, Hkv
    (1, 1, 4, 1),
    (2, 33, 8, 2),
    (2, 64, 8, 2),
    (1, 100, 16, 4),
    (2, 257, 8, 2),
    (1, 300, 4, 4),
    (1, 190, 8, 4),
    (1, 129, 16, 2),
    (2, 520, 32, 8),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}-S{}-{}x{}".format(*c))
def test_prefill_small_shapes(gpu_lib, case):
    B, S, hq, hkv = case
    print(f"[prefill] small {case}", flush=True)
    x = synth.prefill_inputs(B, S, hq, hkv, 128, 16, seed=S + hq + 10 * hkv, device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    out = _run(gpu_lib, x)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", f"prefill {case}")
    _check_append(x, kb, vb)


def test_prefill_row0_is_v0_and_identical_keys_give_running_mean(gpu_lib):
    print("[prefill] closed forms", flush=True)
    x = synth.prefill_inputs(1, 130, 8, 2, 128, 16, seed=4, device=DEV)
    x.k[:] = 0.25  # identical keys: row i = mean of V[0..i]
    out = _run(gpu_lib, x)
    v = to_f64(x.v)
    # row 0 sees one key: exactly V[0] (p = 1, l = 1)
    for h in range(8):
        assert torch.equal(out[0, 0, h].cpu(), x.v[0, 0, h // 4].cpu())
    running = np.cumsum(v[0], axis=0) / np.arange(1, 131)[:, None, None]
    want = np.repeat(running, 4, axis=1)
    assert_close(out[0], want, "bf16", "running mean")


@pytest.fixture(scope="module")
def cfg3():
    x = synth.config3(device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    return x, kb, vb


def test_config3_prefill_whole_output_and_append(gpu_lib, cfg3):
    """Workload 3 at full size (B=4, S=2048, Hq=32, Hkv=8, the launch the benchmark times):
    every (b, head) row of the output against the float64 oracle, and the whole append."""
    print("[prefill] config3 whole output", flush=True)
    x, kb, vb = cfg3
    out = _run(gpu_lib, x)
    _check_append(x, kb, vb)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", "config3 whole output")


@pytest.mark.parametrize("hkv", [32, 16])
def test_prefill_full_size_small_groups_whole_output(gpu_lib, hkv):
    """B=4, S=2048, Hq=32 with G = 1 and G = 2 (the kernels that stream their Q rows, output
    and append with the nt hint): every head against the oracle, the whole append, and a
    bit-identical second call."""
    print(f"[prefill] full size Hkv={hkv}", flush=True)
    x = synth.prefill_inputs(4, 2048, 32, hkv, 128, 16, seed=4000 + hkv, device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    out = _run(gpu_lib, x)
    _check_append(x, kb, vb)
    again = _run(gpu_lib, x)
    assert torch.equal(out, again), "a second call differs"
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", f"prefill full size Hkv={hkv}")


def test_prefill_long_sequence_whole_output(gpu_lib):
    """S = 8192 (4x the benchmark length: 128 key tiles for the last q-tile, the running max
    raised many times): every head against the oracle, and the append of all 8192 positions."""
    print("[prefill] S=8192", flush=True)
    x = synth.prefill_inputs(1, 8192, 8, 2, 128, 16, seed=8192, device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    out = _run(gpu_lib, x)
    _check_append(x, kb, vb)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", "prefill S=8192 whole output")


def test_config3_deterministic(gpu_lib, cfg3):
    print("[prefill] config3 determinism", flush=True)
    x, _, _ = cfg3
    a = _run(gpu_lib, x)
    b = _run(gpu_lib, x)
    assert torch.equal(a, b)
    assert torch.isfinite(a.float()).all()


@pytest.mark.parametrize("scale", [-0.0884, 0.5, 0.0])
def test_prefill_scale_sign_and_magnitude(gpu_lib, scale):
    """The row max is taken on unscaled scores and the scale applied in the exponent;
    a negative scale (max becomes min), a large one (sharp softmax, many rescales) and
    zero (uniform weights, the running mean of V) must all match the oracle."""
    print(f"[prefill] scale {scale}", flush=True)
    x = synth.prefill_inputs(2, 200, 8, 2, 128, 16, seed=77, device=DEV)
    x.scale = scale
    out = _run(gpu_lib, x)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, scale)
    assert_close(out, ref, "bf16", f"prefill scale={scale}")


def test_prefill_more_kv_pairs_than_compute_units(gpu_lib):
    """B * Hkv = 264 (b, kv head) pairs: more than one workgroup per compute unit, so each
    workgroup walks every q-tile of its pair; full output and append against the oracle."""
    print("[prefill] 264 pairs", flush=True)
    x = synth.prefill_inputs(66, 96, 16, 4, 128, 16, seed=264, device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    out = _run(gpu_lib, x)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", "prefill 264 pairs")
    _check_append(x, kb, vb)


@pytest.mark.parametrize("B,S,hq,hkv", [(8, 640, 64, 8), (16, 1100, 8, 2), (16, 600, 16, 8),
                                         (32, 700, 4, 4)])
def test_prefill_several_q_tiles_per_workgroup(gpu_lib, B, S, hq, hkv):
    """More q-tiles than workgroups per (b, kv head) pair on a 256-CU device: every
    workgroup processes several q-tiles in a row (G = 8, 4, 2, 1; the last round only partly
    filled, S not a multiple of the q-tile); the whole output against the oracle, the whole
    append bit for bit."""
    print(f"[prefill] several items B={B} S={S} {hq}x{hkv}", flush=True)
    x = synth.prefill_inputs(B, S, hq, hkv, 128, 16, seed=B * S + hq, device=DEV)
    kb, vb = x.k_cache.cpu(), x.v_cache.cpu()
    out = _run(gpu_lib, x)
    _check_append(x, kb, vb)
    c = x.to("cpu")
    ref = oracle.prefill_causal(c.q, c.k, c.v, c.scale)
    assert_close(out, ref, "bf16", f"prefill several items B={B} S={S}")
