"""Float64 oracle for paged GQA decode over an 8-bit floating-point KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the product.

The pages quote FP8 KV caches as a further halving of decode bytes ([GQA-BATCH], the
performance discussion after section "核心参数调优：PackGQA与NumSplits的协同舞蹈"; [TRT-GQA]
section "显存带宽瓶颈下的理性妥协") but fix no format. Readings (also in the design notes):
  * the two 8-bit formats are the common ones, E4M3 (4 exponent bits, bias 7, 3 mantissa
    bits, no infinities, S.1111.111 is NaN, largest finite 448) and E5M2 (5 exponent bits,
    bias 15, 2 mantissa bits, IEEE-style infinities and NaNs); the decoders below write
    those definitions out bit by bit;
  * one scale per cache tensor: the value of a byte x in the K cache is k_scale * fp8(x)
    (same for V); q stays in bf16/fp32; all arithmetic is exact float64 here;
  * the attention itself is the plain decode definition of ``oracle.attention``.
"""

from __future__ import annotations

import numpy as np

from .attention import decode_paged


def decode_e4m3(x) -> np.ndarray:
    """float64 value of E4M3 bytes (uint8 array): sign, exponent field e (bias 7), mantissa
    m: e == 0 -> (-1)^s * m/8 * 2^-6 (subnormal); e == 15 and m == 7 -> NaN; otherwise
    (-1)^s * (1 + m/8) * 2^(e-7)."""
    x = np.asarray(x, dtype=np.uint8).astype(np.int64)
    s = np.where(x >> 7, -1.0, 1.0)
    e = (x >> 3) & 15
    m = (x & 7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = s * val
    return np.where((e == 15) & (m == 7), np.nan, val)


def decode_e5m2(x) -> np.ndarray:
    """float64 value of E5M2 bytes: exponent field e (bias 15), mantissa m: e == 0 ->
    (-1)^s * m/4 * 2^-14; e == 31 -> +-inf (m == 0) or NaN; otherwise
    (-1)^s * (1 + m/4) * 2^(e-15)."""
    x = np.asarray(x, dtype=np.uint8).astype(np.int64)
    s = np.where(x >> 7, -1.0, 1.0)
    e = (x >> 2) & 31
    m = (x & 3).astype(np.float64)
    val = np.where(e == 0, m / 4.0 * 2.0 ** -14, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return s * val


DECODERS = {"e4m3": decode_e4m3, "e5m2": decode_e5m2}


def dequantize(cache_bytes, scale: float, fmt: str) -> np.ndarray:
    """Value of every cache byte: scale * fp8(byte), float64, same shape."""
    try:
        import torch
        if isinstance(cache_bytes, torch.Tensor):
            cache_bytes = cache_bytes.detach().to("cpu").view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return float(scale) * DECODERS[fmt](cache_bytes)


def decode_paged_fp8(q, k_bytes, v_bytes, k_scale: float, v_scale: float, page_table,
                     context_lens, scale: float, fmt: str) -> np.ndarray:
    """Decode over an 8-bit KV pool: the plain decode definition on the dequantized cache."""
    return decode_paged(q, dequantize(k_bytes, k_scale, fmt), dequantize(v_bytes, v_scale, fmt),
                        page_table, context_lens, scale)
