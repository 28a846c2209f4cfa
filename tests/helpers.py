"""Shared tolerance checks for GPU-vs-oracle parity tests.

Tolerances: float32 paths must match the float64 oracle to max |err| <= 1e-5;
bf16 paths to max |err| <= 2e-2 and relative L2 error <= 5e-3 over the whole
compared output.
"""

import numpy as np
import torch

F32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def to_f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    g = to_f64(got)
    r = to_f64(ref)
    diff = g - r
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(r.ravel()))
    rel = float(np.linalg.norm(diff.ravel())) / denom if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_close(got, ref, dtype, what=""):
    g = to_f64(got)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    max_abs, rel = errors(g, ref)
    if dtype in ("f32", torch.float32):
        assert max_abs <= F32_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {F32_MAX_ABS}"
    else:
        assert max_abs <= BF16_MAX_ABS, f"{what}: max abs {max_abs:.3e} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel L2 {rel:.3e} > {BF16_REL_L2}"
    return max_abs, rel
