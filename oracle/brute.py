"""Pure-Python brute-force attention on tiny inputs: TEST INFRASTRUCTURE ONLY.

Scalar loops over nested lists of Python floats, ``math.exp`` and
``math.fsum`` only (no numpy, no torch), written independently of
``oracle.attention`` so that the two can pin each other. Same definition and
readings: out = softmax(scale * q K^T) V with [TRT-GQA] contiguous head
grouping ("技术演进背景"), page-table addressing ([TRT-GQA]
"动态形状与KV Cache管理", [TRTLLM-OPS] section 4.2.2) and the causal mask of
[GQA-BATCH] Figure 2 (row i sees keys 0..i).
"""

from __future__ import annotations

import math


def _softmax_avg(scores, values):
    """sum_t softmax(scores)_t * values[t] (values: list of equal-length lists)."""
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    z = math.fsum(w)
    d = len(values[0])
    return [math.fsum(w[t] * values[t][c] for t in range(len(w))) / z for c in range(d)]


def decode(q, k_pool, v_pool, page_table, context_lens, scale):
    """q[b][h][c]; pools[page][kvh][slot][c]; page_table[b][i]; -> out[b][h][c]."""
    B = len(q)
    hq = len(q[0])
    hkv = len(k_pool[0])
    group = hq // hkv
    page = len(k_pool[0][0])
    d = len(q[0][0])
    out = []
    for b in range(B):
        T = context_lens[b]
        row = []
        for h in range(hq):
            g = h // group
            if T == 0:
                row.append([0.0] * d)
                continue
            keys, vals = [], []
            for t in range(T):
                p = page_table[b][t // page]
                s = t % page
                keys.append(k_pool[p][g][s])
                vals.append(v_pool[p][g][s])
            scores = [scale * math.fsum(q[b][h][c] * keys[t][c] for c in range(d))
                      for t in range(T)]
            row.append(_softmax_avg(scores, vals))
        out.append(row)
    return out


def prefill(q, k, v, scale):
    """q[b][i][h][c], k/v[b][j][kvh][c]; row i attends j <= i -> out[b][i][h][c]."""
    B = len(q)
    S = len(q[0])
    hq = len(q[0][0])
    hkv = len(k[0][0])
    group = hq // hkv
    d = len(q[0][0][0])
    out = []
    for b in range(B):
        rows = []
        for i in range(S):
            heads = []
            for h in range(hq):
                g = h // group
                scores = [scale * math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d))
                          for j in range(i + 1)]
                heads.append(_softmax_avg(scores, [v[b][j][g] for j in range(i + 1)]))
            rows.append(heads)
        out.append(rows)
    return out


def prefill_paged(q, k_pool, v_pool, k_new, v_new, page_table, past, new, scale):
    """Chunked prefill on nested lists: sequence b holds past[b] cached tokens (pools
    [page][kvh][slot][c] through page_table[b]) and appends new[b] tokens k_new/v_new[b][i];
    new row i (position past[b] + i) attends keys 0..past[b]+i. -> out[b][i][h][c] for
    i < new[b]."""
    B = len(q)
    hq = len(q[0][0])
    hkv = len(k_new[0][0])
    group = hq // hkv
    page = len(k_pool[0][0])
    d = len(q[0][0][0])
    out = []
    for b in range(B):
        rows = []
        for i in range(new[b]):
            heads = []
            for h in range(hq):
                g = h // group
                keys, vals = [], []
                for j in range(past[b] + i + 1):
                    if j < past[b]:
                        p = page_table[b][j // page]
                        keys.append(k_pool[p][g][j % page])
                        vals.append(v_pool[p][g][j % page])
                    else:
                        keys.append(k_new[b][j - past[b]][g])
                        vals.append(v_new[b][j - past[b]][g])
                scores = [scale * math.fsum(q[b][i][h][c] * keys[t][c] for c in range(d))
                          for t in range(len(keys))]
                heads.append(_softmax_avg(scores, vals))
            rows.append(heads)
        out.append(rows)
    return out
