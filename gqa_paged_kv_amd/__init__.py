"""Python binding of libgqa (paged GQA attention for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gqa.h``. PyTorch provides the
device memory (outputs and split workspace are allocated with torch) and the
current stream. There is no fallback: if ``libgqa.so`` is missing or a call
fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgqa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_LAUNCH, ERR_SCRATCH = 0, 1, 2, 3, 4
F32, BF16, FP8_E4M3, FP8_E5M2 = 0, 1, 2, 3
_FP8_CODE = {"e4m3": FP8_E4M3, "e5m2": FP8_E5M2}
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16}

# Exported symbols and their C signatures (argument types in order).
_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "gqa_decode_paged": (_i, [_p, _p, _p, _p, _p, _p, _p, _p] + [_i] * 8 + [_f, _i, _p]),
    "gqa_decode_paged_balanced": (_i, [_p] * 7 + [_sz] + [_i] * 7 + [_f, _i, _p]),
    "gqa_decode_paged_balanced_noalloc": (_i, [_p] * 6 + [_i] * 7 + [_f, _i, _p]),
    "gqa_decode_balanced_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "gqa_decode_append": (_i, [_p] * 9 + [_sz] + [_i] * 7 + [_f, _i, _p]),
    "gqa_decode_paged_fp8": (_i, [_p, _p, _p, _f, _f, _p, _p, _p, _p, _sz] + [_i] * 7 + [_f, _i, _p]),
    "gqa_prefill_causal": (_i, [_p] * 7 + [_i] * 8 + [_f, _i, _p]),
    "gqa_prefill_paged": (_i, [_p] * 9 + [_i] * 8 + [_f, _i, _p]),
    "gqa_combine_splits": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "gqa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "gqa_status_string": (ctypes.c_char_p, [_i]),
    "gqa_validate_decode": (_i, [_p] * 8 + [_i] * 8 + [_f, _i]),
    "gqa_validate_decode_fp8": (_i, [_p, _p, _p, _f, _f, _p, _p, _p] + [_i] * 7 + [_f, _i]),
    "gqa_validate_prefill": (_i, [_p] * 7 + [_i] * 8 + [_f, _i]),
    "gqa_validate_prefill_paged": (_i, [_p] * 9 + [_i] * 8 + [_f, _i]),
    "gqa_validate_combine": (_i, [_p, _p, _p, _i, _i, _i, _i, _i]),
    "gqa_gather_paged": (_i, [_p, _p, _p, _p] + [_i] * 7 + [_p]),
    "gqa_decode_balanced_route": (_i, [_i, _i, _i, _i, _i, _sz]),
    "gqa_check_page_table": (_i, [_p, _p, _i, _i, _i, _i]),
    "gqa_bench_stream_read": (_i, [_p, _sz, _p, _i, _i, _p]),
    "gqa_bench_flush_read": (_i, [_p, _sz, _p, _p]),
    "gqa_bench_mfma_bf16": (_i, [_p, _i, _i, _p]),
}

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqa.so (built by ``gqa_paged_kv_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gqa_paged_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (ret, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = ret
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gqa_status_string(status).decode()


def workspace_bytes(B: int, Hq: int, D: int, num_splits: int) -> int:
    return int(load().gqa_decode_workspace_bytes(B, Hq, D, num_splits))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(st: int, what: str):
    if st != OK:
        raise GQAError(st, what)


def _need(t: torch.Tensor, name: str, dtype=None, dim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions")


def alloc_workspace(B: int, Hq: int, D: int, num_splits: int, device):
    """fp32 split workspace (ws_o [B][Hq][NS][D], ws_lse [B][Hq][NS])."""
    ws_o = torch.empty((B, Hq, num_splits, D), dtype=torch.float32, device=device)
    ws_lse = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=device)
    return ws_o, ws_lse


def decode_paged(q, k_cache, v_cache, page_table, context_lens, num_splits: int = 1,
                 scale: float | None = None, out=None, workspace=None):
    """Paged GQA decode; returns out [B][Hq][D] in q's dtype (enqueued on the current stream)."""
    lib = load()
    _need(q, "q", dim=3)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype, 3)
    ws_o = ws_lse = None
    if num_splits > 1:
        if workspace is None:
            workspace = alloc_workspace(B, Hq, D, num_splits, q.device)
        ws_o, ws_lse = workspace
        _need(ws_o, "ws_o", torch.float32)
        _need(ws_lse, "ws_lse", torch.float32)
        if ws_o.numel() < B * Hq * num_splits * D or ws_lse.numel() < B * Hq * num_splits:
            raise ValueError("workspace too small")
    st = lib.gqa_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                              _ptr(context_lens), _ptr(out), _ptr(ws_o), _ptr(ws_lse), B, Hq, Hkv,
                              D, P, page_table.shape[1], num_pages, num_splits, scale,
                              _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "gqa_decode_paged")
    return out


# Leading bytes of a balanced-decode workspace that hold counters (zero before first use;
# every completed call leaves them zero, every call tags them with a new epoch).
BALANCED_WS_RESERVED = 98304


def balanced_workspace(B: int, Hq: int, Hkv: int, D: int, device):
    """Device scratch for decode_paged_balanced / decode_append / decode_paged_fp8 (uint8
    tensor, 256-byte aligned, zero-filled: its leading counters must start at zero; every
    completed call leaves them zero, so the tensor can be reused by calls enqueued in order)."""
    n = int(load().gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D))
    return torch.zeros(n, dtype=torch.uint8, device=device)


def decode_paged_balanced(q, k_cache, v_cache, page_table, context_lens,
                          scale: float | None = None, out=None, workspace=None):
    """Paged GQA decode with the library's balanced work partition; returns out [B][Hq][D]."""
    lib = load()
    _need(q, "q", dim=3)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", q.dtype, 3)
    if workspace is None:
        workspace = balanced_workspace(B, Hq, Hkv, D, q.device)
    _need(workspace, "workspace")
    st = lib.gqa_decode_paged_balanced(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
                                       _ptr(context_lens), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), B, Hq, Hkv,
                                       D, P, page_table.shape[1], num_pages, scale,
                                       _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "gqa_decode_paged_balanced")
    return out


# Bytes of the static device buffer behind decode_paged_balanced_noalloc.
NOALLOC_SCRATCH_BYTES = 34701312


def decode_paged_balanced_noalloc(q, k_cache, v_cache, page_table, context_lens, out,
                                  scale: float | None = None):
    """decode_paged_balanced on the library's static device scratch (no workspace argument;
    the C entry point allocates nothing). ``out`` [B][Hq][D] must be given; it is returned."""
    lib = load()
    _need(q, "q", dim=3)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(out, "out", q.dtype, 3)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or out.shape != q.shape:
        raise ValueError("shapes do not match q")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    st = lib.gqa_decode_paged_balanced_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                               _ptr(page_table), _ptr(context_lens), _ptr(out),
                                               B, Hq, Hkv, D, P, page_table.shape[1], num_pages,
                                               scale, _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "gqa_decode_paged_balanced_noalloc")
    return out


def combine_splits(ws_o, ws_lse, out_dtype=torch.bfloat16, out=None):
    """LSE merge of split partials; returns out [B][Hq][D]."""
    lib = load()
    _need(ws_o, "ws_o", torch.float32, 4)
    _need(ws_lse, "ws_lse", torch.float32, 3)
    B, Hq, ns, D = ws_o.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype, device=ws_o.device)
    st = lib.gqa_combine_splits(_ptr(ws_o), _ptr(ws_lse), _ptr(out), B, Hq, D, ns,
                                _DTYPE_CODE[out.dtype], _stream(ws_o.device))
    _check(st, "gqa_combine_splits")
    return out


def decode_append(q, k_new, v_new, k_cache, v_cache, page_table, context_lens,
                  scale: float | None = None, out=None, workspace=None):
    """One decode step with its own token: k_new / v_new [B][Hkv][D] are written at position
    context_lens[b] of each sequence, which then attends context_lens[b] + 1 tokens (the new
    one included). context_lens is not changed. Returns out [B][Hq][D]."""
    lib = load()
    _need(q, "q", dim=3)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _need(k_new, "k_new", q.dtype, 3)
    _need(v_new, "v_new", q.dtype, 3)
    _need(k_cache, "k_cache", q.dtype, 4)
    _need(v_cache, "v_cache", q.dtype, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or k_new.shape != (B, Hkv, D) or \
            v_new.shape != k_new.shape:
        raise ValueError("shapes do not match")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = balanced_workspace(B, Hq, Hkv, D, q.device)
    st = lib.gqa_decode_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                               _ptr(page_table), _ptr(context_lens), _ptr(out), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), B, Hq, Hkv, D, P,
                               page_table.shape[1], num_pages, scale, _DTYPE_CODE[q.dtype],
                               _stream(q.device))
    _check(st, "gqa_decode_append")
    return out


def decode_paged_fp8(q, k_cache, v_cache, k_scale: float, v_scale: float, page_table,
                     context_lens, fmt: str = "e4m3", scale: float | None = None, out=None,
                     workspace=None):
    """Paged GQA decode over an 8-bit KV pool (uint8 bytes in format ``fmt``, "e4m3" or
    "e5m2"; element value = scale * fp8(byte)); q and out bf16; returns out [B][Hq][D]."""
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.uint8, 4)
    _need(v_cache, "v_cache", torch.uint8, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if fmt not in _FP8_CODE:
        raise ValueError(f"unknown 8-bit format {fmt}")
    B, Hq, D = q.shape
    num_pages, Hkv, P, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if page_table.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("page_table / context_lens batch mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _need(out, "out", torch.bfloat16, 3)
    if workspace is None:
        workspace = balanced_workspace(B, Hq, Hkv, D, q.device)
    _need(workspace, "workspace")
    st = lib.gqa_decode_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), float(k_scale),
                                  float(v_scale), _ptr(page_table), _ptr(context_lens), _ptr(out),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  B, Hq, Hkv, D, P, page_table.shape[1], num_pages, scale,
                                  _FP8_CODE[fmt], _stream(q.device))
    _check(st, "gqa_decode_paged_fp8")
    return out


def prefill_causal(q, k, v, k_cache, v_cache, page_table, scale: float | None = None, out=None):
    """Causal GQA prefill; appends k/v into the paged cache; returns out [B][S][Hq][D]."""
    lib = load()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(page_table, "page_table", torch.int32, 2)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    num_pages, Hkv_c, P, Dc = k_cache.shape
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or Hkv_c != Hkv or Dc != D:
        raise ValueError("prefill shapes do not match")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    st = lib.gqa_prefill_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                _ptr(page_table), _ptr(out), B, S, Hq, Hkv, D, P,
                                page_table.shape[1], num_pages, scale, BF16, _stream(q.device))
    _check(st, "gqa_prefill_causal")
    return out


def prefill_paged(q, k, v, k_cache, v_cache, page_table, past_lens, new_lens,
                  scale: float | None = None, out=None):
    """Chunked prefill: sequence b holds past_lens[b] cached tokens and appends new_lens[b]
    tokens (k/v rows) at positions past .. past+new-1; new row i attends keys 0..past+i.
    Returns out [B][S][Hq][D] (rows i >= new_lens[b] untouched)."""
    lib = load()
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(page_table, "page_table", torch.int32, 2)
    _need(past_lens, "past_lens", torch.int32, 1)
    _need(new_lens, "new_lens", torch.int32, 1)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    num_pages, Hkv_c, P, Dc = k_cache.shape
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or Hkv_c != Hkv or Dc != D:
        raise ValueError("prefill shapes do not match")
    if past_lens.shape != (B,) or new_lens.shape != (B,):
        raise ValueError("past_lens / new_lens must be [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    st = lib.gqa_prefill_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                               _ptr(page_table), _ptr(past_lens), _ptr(new_lens), _ptr(out), B, S,
                               Hq, Hkv, D, P, page_table.shape[1], num_pages, scale, BF16,
                               _stream(q.device))
    _check(st, "gqa_prefill_paged")
    return out


def gather_paged(cache, page_table, context_lens, dst=None):
    """Test helper: contiguous copy [B][max_pages*P][Hkv][D] of the live tokens."""
    lib = load()
    _need(cache, "cache", None, 4)
    num_pages, Hkv, P, D = cache.shape
    B, max_pages = page_table.shape
    if dst is None:
        dst = torch.zeros((B, max_pages * P, Hkv, D), dtype=cache.dtype, device=cache.device)
    st = lib.gqa_gather_paged(_ptr(cache), _ptr(page_table), _ptr(context_lens), _ptr(dst), B,
                              Hkv, D, P, max_pages, num_pages, _DTYPE_CODE[cache.dtype],
                              _stream(cache.device))
    _check(st, "gqa_gather_paged")
    return dst


def balanced_route(B: int, Hq: int, Hkv: int, D: int, max_pages: int,
                   workspace_bytes: int | None = None) -> int:
    """Route of decode_paged_balanced: 0 = persistent kernel, n >= 1 = split path with n splits
    (host-only; workspace_bytes defaults to the size balanced_workspace allocates)."""
    lib = load()
    if workspace_bytes is None:
        workspace_bytes = int(lib.gqa_decode_balanced_workspace_bytes(B, Hq, Hkv, D))
    return int(lib.gqa_decode_balanced_route(B, Hq, Hkv, D, max_pages, workspace_bytes))


def check_page_table(page_table, tokens, num_pages: int, page_size: int = 16) -> int:
    """Host check of the page ids a call would touch (see gqa_check_page_table): page_table
    [B][max_pages] and tokens [B] (int32, any device; copied to the host). Returns the status."""
    pt = page_table.detach().to("cpu", torch.int32).contiguous()
    tk = torch.as_tensor(tokens).detach().to("cpu", torch.int32).contiguous()
    B, max_pages = pt.shape
    if tk.shape != (B,):
        raise ValueError("tokens must be [B]")
    return int(load().gqa_check_page_table(_ptr(pt), _ptr(tk), B, max_pages, page_size,
                                           num_pages))


def bench_stream_read(src, sink, blocks_per_cu: int = 8, unroll: int = 8):
    """Bench-only: stream-read all of ``src`` (a device tensor) with 128-bit loads."""
    st = load().gqa_bench_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                      blocks_per_cu, unroll, _stream(src.device))
    _check(st, "gqa_bench_stream_read")


def bench_flush_read(src, sink):
    """Bench-only: read all of ``src`` with ordinary loads (evicts the L2s and the Infinity
    Cache when ``src`` is several times their size)."""
    st = load().gqa_bench_flush_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                     _stream(src.device))
    _check(st, "gqa_bench_flush_read")


def bench_mfma_bf16(sink, blocks: int, iters: int):
    """Bench-only: back-to-back bf16 32x32x16 MFMAs; flops = blocks * 8 * iters * 32768."""
    st = load().gqa_bench_mfma_bf16(_ptr(sink), blocks, iters, _stream(sink.device))
    _check(st, "gqa_bench_mfma_bf16")
