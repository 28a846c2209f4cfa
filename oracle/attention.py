"""Float64 oracle for paged GQA decode, split/combine and causal prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the product.

Every function evaluates the plain definition of attention,
``softmax(scale * q K^T) V`` ([TRTLLM-OPS] section 4.1, the unfused
Q*K^T -> Softmax -> x V decomposition), with no tiling, no online softmax and
no fusion: the fused/tiled/split GPU method reaches exactly this result in
exact arithmetic ([TRTLLM-OPS] section 4.2.1 only changes where intermediates
live). K/V rows are fetched one logical token at a time through the page
table ([TRT-GQA] section "动态形状与KV Cache管理"; [TRTLLM-OPS] section 4.2.2).

Readings (the pages leave these open):
  * head grouping is contiguous: query head h uses KV head h // G with
    G = Hq / Hkv, i.e. repeat_kv repeats every KV head G times in a row
    ([TRT-GQA] sections "技术演进背景" and "图优化与算子融合");
  * the scale is an explicit argument (callers pass 1/sqrt(D));
  * the page pool is [num_pages][Hkv][P][D]: token t of sequence b lives in
    physical page PT[b][t // P], slot t % P, of the (page, kv-head) block;
  * decode's single query attends every cached token 0..T_b-1 (no mask);
    T_b = 0 gives a zero output;
  * prefill row i attends keys 0..i (causal, diagonal included), the new
    tokens being positions 0..S-1 ([GQA-BATCH] Figure 2 caption names the
    causal mask, nothing more);
  * chunked prefill (a chunk of n_b new tokens appended to a sequence that
    already holds p_b cached tokens; [TRT-GQA] section "动态形状与KV Cache管理"
    has the cache grow by the new tokens) puts new row i at absolute position
    p_b + i; it attends every cached key and the new keys up to itself
    (keys 0..p_b+i: the causal mask of [GQA-BATCH] Figure 2 aligned to the
    bottom-right corner); the new K/V rows are written at positions
    p_b..p_b+n_b-1 before they are read;
  * NumSplits ([GQA-BATCH] section "核心参数调优") splits a sequence's pages
    into NS contiguous page ranges of ceil(np/NS) pages; each split yields a
    normalised partial output and a natural-log log-sum-exp; an empty split
    has lse = -inf and a zero output.
"""

from __future__ import annotations

import math

import numpy as np

try:  # torch is only needed to widen bfloat16 tensors exactly.
    import torch
except Exception:  # pragma: no cover - torch is present in this environment
    torch = None


def _f64(x) -> np.ndarray:
    """Widen a tensor/array to float64 exactly (bf16 and fp32 embed in fp64)."""
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head used by query head ``h`` under contiguous grouping.

    [TRT-GQA] section "技术演进背景": query heads are split into groups and each
    group shares one K/V head; repeat_kv ("图优化与算子融合") expands K/V "to
    match Q". Reading: group g holds query heads g*G .. g*G+G-1.
    """
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


def logical_to_physical(page_table_row, t: int, page_size: int):
    """(physical page, slot) holding logical token ``t`` of one sequence.

    [TRT-GQA] section "动态形状与KV Cache管理": the caller passes the physical
    page indices and the logical position is mapped to a physical address;
    [TRTLLM-OPS] section 4.2.2: fixed-size pages, logically contiguous tokens
    may sit in scattered physical pages, a page table maps between them.
    """
    return int(page_table_row[t // page_size]), t % page_size


def kv_bytes(tokens: int, hkv: int, head_dim: int, elem_bytes: int) -> int:
    """Bytes of one K cache plus one V cache holding ``tokens`` tokens.

    [TRT-GQA] section "技术演进背景": every KV head caches one K row and one V
    row per token, so the cache scales with the KV-head count (32 heads in 8
    groups keep 8 K/V heads: 1/4 of MHA).
    """
    return 2 * tokens * hkv * head_dim * elem_bytes


def gather_paged(cache, page_table, context_lens, page_size: int):
    """Per-sequence contiguous copy of a paged cache: list of [T_b][Hkv][D].

    Token by token through ``logical_to_physical``; the dtype is preserved
    (this is a copy, compared bit for bit).
    """
    pt = _i64(page_table)
    lens = _i64(context_lens)
    out = []
    for b in range(pt.shape[0]):
        rows = []
        for t in range(int(lens[b])):
            p, s = logical_to_physical(pt[b], t, page_size)
            rows.append(cache[p, :, s, :])
        if rows:
            out.append(torch.stack(rows, 0) if torch is not None and isinstance(cache, torch.Tensor)
                       else np.stack(rows, 0))
        else:
            shape = (0, cache.shape[1], cache.shape[3])
            out.append(cache.new_empty(shape) if torch is not None and isinstance(cache, torch.Tensor)
                       else np.empty(shape, dtype=cache.dtype))
    return out


def _gather_rows(cache, pt_row, n_tokens: int, kvh: int, page_size: int) -> np.ndarray:
    """[n_tokens][D] float64 rows of one (sequence, kv head), via the page table."""
    if n_tokens == 0:
        return np.zeros((0, cache.shape[3]), dtype=np.float64)
    t = np.arange(n_tokens)
    pages = np.asarray([int(pt_row[i]) for i in (t // page_size)], dtype=np.int64)
    slots = t % page_size
    if torch is not None and isinstance(cache, torch.Tensor):
        rows = cache[torch.from_numpy(pages), kvh, torch.from_numpy(slots), :]
    else:
        rows = cache[pages, kvh, slots, :]
    return _f64(rows)


def _softmax_weighted_sum(scores: np.ndarray, v: np.ndarray) -> np.ndarray:
    """softmax(scores) @ v for 1-D scores (max subtracted: same value exactly)."""
    m = scores.max()
    w = np.exp(scores - m)
    return (w @ v) / w.sum()


def decode_paged_rows(q, k_cache, v_cache, page_table, context_lens, scale: float,
                      rows):
    """Decode outputs for the (b, h) pairs in ``rows`` only: dict -> [D] float64.

    Lets large workloads be checked on a sample of outputs.
    """
    pt = _i64(page_table)
    lens = _i64(context_lens)
    B, hq, d = q.shape
    hkv = k_cache.shape[1]
    page_size = k_cache.shape[2]
    res = {}
    last_key, K, V = None, None, None  # rows of the last (b, kv head) gathered
    for (b, h) in rows:
        kvh = kv_head_of(h, hq, hkv)
        T = int(lens[b])
        if T == 0:
            res[(b, h)] = np.zeros(d)
            continue
        if (b, kvh) != last_key:
            last_key = (b, kvh)
            K = _gather_rows(k_cache, pt[b], T, kvh, page_size)
            V = _gather_rows(v_cache, pt[b], T, kvh, page_size)
        qv = _f64(q[b, h])
        scores = scale * (K @ qv)
        res[(b, h)] = _softmax_weighted_sum(scores, V)
    return res


def decode_paged(q, k_cache, v_cache, page_table, context_lens, scale: float) -> np.ndarray:
    """Single-token paged GQA decode: out[b][h] = softmax(scale q K_b^T) V_b.

    q [B][Hq][D]; k_cache, v_cache [num_pages][Hkv][P][D]; page_table
    [B][max_pages]; context_lens [B]. Returns [B][Hq][D] float64.
    """
    B, hq, d = q.shape
    rows = [(b, h) for b in range(B) for h in range(hq)]
    got = decode_paged_rows(q, k_cache, v_cache, page_table, context_lens, scale, rows)
    out = np.zeros((B, hq, d))
    for (b, h), o in got.items():
        out[b, h] = o
    return out


def split_page_ranges(n_pages: int, num_splits: int):
    """Logical page range [start, end) of every split of one sequence.

    [GQA-BATCH] section "核心参数调优": NumSplits cuts the attention computation
    into sub-problems. Reading: split s covers pages [s*c, min((s+1)*c, n)) with
    c = ceil(n / NS); later splits may be empty.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    c = -(-n_pages // num_splits) if n_pages > 0 else 0
    ranges = []
    for s in range(num_splits):
        lo = min(s * c, n_pages)
        hi = min((s + 1) * c, n_pages)
        ranges.append((lo, hi))
    return ranges


def decode_split_partials(q, k_cache, v_cache, page_table, context_lens, scale: float,
                          num_splits: int):
    """Per-split normalised partial outputs and natural-log LSEs.

    Returns (o [B][Hq][NS][D], lse [B][Hq][NS]) float64 where, over the tokens
    of split s, o = sum_t w_t V_t / sum_t w_t and lse = log sum_t exp(score_t);
    an empty split gives o = 0, lse = -inf.
    """
    pt = _i64(page_table)
    lens = _i64(context_lens)
    B, hq, d = q.shape
    hkv = k_cache.shape[1]
    page_size = k_cache.shape[2]
    o = np.zeros((B, hq, num_splits, d))
    lse = np.full((B, hq, num_splits), -np.inf)
    for b in range(B):
        T = int(lens[b])
        n_pages = -(-T // page_size)
        for kvh in range(hkv):
            K = _gather_rows(k_cache, pt[b], T, kvh, page_size)
            V = _gather_rows(v_cache, pt[b], T, kvh, page_size)
            for h in range(kvh * (hq // hkv), (kvh + 1) * (hq // hkv)):
                qv = _f64(q[b, h])
                for s, (lo, hi) in enumerate(split_page_ranges(n_pages, num_splits)):
                    t0, t1 = lo * page_size, min(hi * page_size, T)
                    if t1 <= t0:
                        continue
                    scores = scale * (K[t0:t1] @ qv)
                    m = scores.max()
                    w = np.exp(scores - m)
                    o[b, h, s] = (w @ V[t0:t1]) / w.sum()
                    lse[b, h, s] = m + math.log(w.sum())
    return o, lse


def combine_splits(o, lse) -> np.ndarray:
    """Merge split partials: out = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M).

    o [..][NS][D], lse [..][NS] (natural log; -inf marks an empty split);
    M = max_s lse_s; a row whose splits are all empty is zero.
    """
    o = _f64(o)
    lse = _f64(lse)
    lead = lse.shape[:-1]
    out = np.zeros(lead + (o.shape[-1],))
    for idx in np.ndindex(*lead):
        ls = lse[idx]
        M = ls.max()
        if M == -np.inf:
            continue
        w = np.exp(ls - M)
        out[idx] = (w @ o[idx]) / w.sum()
    return out


def prefill_causal_rows(q, k, v, scale: float, rows):
    """Causal prefill outputs for the (b, h) pairs in ``rows``: dict -> [S][D].

    q [B][S][Hq][D]; k, v [B][S][Hkv][D]. Row i attends keys 0..i.
    """
    B, S, hq, d = q.shape
    hkv = k.shape[2]
    mask = np.triu(np.ones((S, S), dtype=bool), k=1)  # key j > query i
    res = {}
    for (b, h) in rows:
        kvh = kv_head_of(h, hq, hkv)
        Q = _f64(q[b, :, h, :])
        K = _f64(k[b, :, kvh, :])
        V = _f64(v[b, :, kvh, :])
        scores = scale * (Q @ K.T)
        scores[mask] = -np.inf
        m = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - m)
        res[(b, h)] = (w @ V) / w.sum(axis=1, keepdims=True)
    return res


def prefill_causal(q, k, v, scale: float) -> np.ndarray:
    """Causal GQA prefill over S new tokens: [B][S][Hq][D] float64."""
    B, S, hq, d = q.shape
    out = np.zeros((B, S, hq, d))
    got = prefill_causal_rows(q, k, v, scale, [(b, h) for b in range(B) for h in range(hq)])
    for (b, h), o in got.items():
        out[b, :, h, :] = o
    return out


def append_paged(cache, new, page_table, page_size: int):
    """Cache after writing ``new`` [B][S][Hkv][D] at logical positions 0..S-1.

    Returns a copy of ``cache`` [num_pages][Hkv][P][D] (same dtype, bit copy)
    with pool[PT[b][j // P]][kvh][j % P] = new[b][j][kvh] for every j < S.
    """
    out = cache.clone() if torch is not None and isinstance(cache, torch.Tensor) else cache.copy()
    pt = _i64(page_table)
    B, S, hkv, _ = new.shape
    for b in range(B):
        for j in range(S):
            p, s = logical_to_physical(pt[b], j, page_size)
            out[p, :, s, :] = new[b, j, :, :]
    return out


def append_paged_at(cache, new, page_table, past_lens, new_lens, page_size: int):
    """Cache after writing new[b][i] at logical position past_lens[b] + i, i < new_lens[b].

    ``new`` is [B][S][Hkv][D]; rows i >= new_lens[b] are ignored. Bit copy, as append_paged.
    """
    out = cache.clone() if torch is not None and isinstance(cache, torch.Tensor) else cache.copy()
    pt = _i64(page_table)
    past = _i64(past_lens)
    nl = _i64(new_lens)
    for b in range(new.shape[0]):
        for i in range(int(nl[b])):
            p, s = logical_to_physical(pt[b], int(past[b]) + i, page_size)
            out[p, :, s, :] = new[b, i, :, :]
    return out


def prefill_paged_rows(q, k_cache, v_cache, k_new, v_new, page_table, past_lens, new_lens,
                       scale: float, rows, page_size: int = 16):
    """Chunked prefill outputs for the (b, h) pairs in ``rows``: dict -> [new_lens[b]][D].

    Sequence b holds past_lens[b] tokens in the paged cache (``k_cache``, ``v_cache`` as
    they were before the chunk; positions < past_lens[b] are read through page_table)
    and appends new_lens[b] tokens whose K/V are k_new[b][:n], v_new[b][:n]. New row i is
    the query at position p + i and attends keys 0..p+i (cached keys, then new keys).
    """
    B, S, hq, d = q.shape
    hkv = k_new.shape[2]
    pt = _i64(page_table)
    past = _i64(past_lens)
    nl = _i64(new_lens)
    res = {}
    for (b, h) in rows:
        p, n = int(past[b]), int(nl[b])
        kvh = kv_head_of(h, hq, hkv)
        K = np.concatenate([_gather_rows(k_cache, pt[b], p, kvh, page_size),
                            _f64(k_new[b, :n, kvh, :])], axis=0)
        V = np.concatenate([_gather_rows(v_cache, pt[b], p, kvh, page_size),
                            _f64(v_new[b, :n, kvh, :])], axis=0)
        Q = _f64(q[b, :n, h, :])
        scores = scale * (Q @ K.T)  # [n][p + n]
        mask = np.arange(p + n)[None, :] > (p + np.arange(n))[:, None]
        scores[mask] = -np.inf
        m = scores.max(axis=1, keepdims=True)
        w = np.exp(scores - m)
        res[(b, h)] = (w @ V) / w.sum(axis=1, keepdims=True)
    return res


def prefill_paged(q, k_cache, v_cache, k_new, v_new, page_table, past_lens, new_lens,
                  scale: float, page_size: int = 16) -> np.ndarray:
    """Chunked prefill: [B][S][Hq][D] float64; rows i >= new_lens[b] are NaN (undefined)."""
    B, S, hq, d = q.shape
    out = np.full((B, S, hq, d), np.nan)
    got = prefill_paged_rows(q, k_cache, v_cache, k_new, v_new, page_table, past_lens,
                             new_lens, scale, [(b, h) for b in range(B) for h in range(hq)],
                             page_size)
    for (b, h), o in got.items():
        out[b, :o.shape[0], h, :] = o
    return out
