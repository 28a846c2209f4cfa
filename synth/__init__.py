"""Seeded synthetic inputs for paged GQA decode and causal prefill.

Shared by the tests, the smoke check and the benchmark, on both sides of the
parity check (the HIP library and the float64 oracle). This module only
*draws and lays out* data: it holds none of the attention arithmetic.

Recipe (fixed draw order from one ``torch.Generator`` per call):
context lengths -> Q -> K pool -> V pool -> page permutation -> hot tokens.
Values are N(0, 1) drawn in float32 and rounded to the storage dtype with
round-to-nearest-even (bf16) or kept as float32.

Pool layout: ``[num_pages][Hkv][P][D]`` for K and for V; sequence b's logical
page i lives at physical page ``page_table[b][i]``. With ``identity=True``
sequence b owns pages ``b*max_pages ...`` in order; otherwise the
``N = sum_b ceil(T_b / P)`` live pages take physical ids from a seeded
permutation of ``range(N)`` in (b, logical page) order. ``pad_pages`` extra
pages follow the live ones. With ``poison=True`` every slot that no live
token owns (the tail of each sequence's last page and all pad pages) holds
NaN, and page-table entries past a sequence's last page hold ``pt_fill``
(default -1): a correct kernel never reads any of them.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B][Hq][D]
    k_cache: torch.Tensor      # [num_pages][Hkv][P][D]
    v_cache: torch.Tensor      # [num_pages][Hkv][P][D]
    page_table: torch.Tensor   # [B][max_pages] int32
    context_lens: torch.Tensor  # [B] int32
    scale: float
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, hq, d = self.q.shape
        return dict(B=B, Hq=hq, Hkv=self.k_cache.shape[1], D=d, P=self.k_cache.shape[2],
                    max_pages=self.page_table.shape[1], num_pages=self.k_cache.shape[0])

    def to(self, device):
        return DecodeInputs(self.q.to(device), self.k_cache.to(device), self.v_cache.to(device),
                            self.page_table.to(device), self.context_lens.to(device),
                            self.scale, dict(self.meta))


@dataclass
class PrefillInputs:
    q: torch.Tensor            # [B][S][Hq][D]
    k: torch.Tensor            # [B][S][Hkv][D]
    v: torch.Tensor            # [B][S][Hkv][D]
    k_cache: torch.Tensor      # [num_pages][Hkv][P][D] (initial contents)
    v_cache: torch.Tensor
    page_table: torch.Tensor   # [B][max_pages] int32
    scale: float
    meta: dict = field(default_factory=dict)

    def to(self, device):
        return PrefillInputs(self.q.to(device), self.k.to(device), self.v.to(device),
                             self.k_cache.to(device), self.v_cache.to(device),
                             self.page_table.to(device), self.scale, dict(self.meta))


def _randn(shape, gen, dtype, device):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device).to(dtype)


def _lens(spec, B, gen):
    if isinstance(spec, int):
        return torch.full((B,), spec, dtype=torch.int64)
    if isinstance(spec, tuple):
        lo, hi = spec  # closed interval
        return torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64)
    lens = torch.as_tensor(list(spec), dtype=torch.int64)
    assert lens.numel() == B
    return lens


def decode_inputs(B, Hq, Hkv, D, P, lens, dtype="bf16", seed=0, *, identity=False,
                  pad_pages=64, poison=True, pt_fill=-1, hot_tokens=0, hot_scale=4.0,
                  max_pages=None, device="cpu"):
    """Paged decode inputs. ``lens``: int (all equal), (lo, hi) closed range or list."""
    dt = DTYPES[dtype]
    dev = torch.device(device)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    dgen = gen if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    ctx = _lens(lens, B, gen)
    n_pages = [(int(t) + P - 1) // P for t in ctx]
    mp = max(max(n_pages), 1) if max_pages is None else max_pages
    assert mp >= max(n_pages)
    live = sum(n_pages) if not identity else B * mp
    num_pages = live + pad_pages
    q = _randn((B, Hq, D), dgen, dt, dev)
    k_cache = _randn((num_pages, Hkv, P, D), dgen, dt, dev)
    v_cache = _randn((num_pages, Hkv, P, D), dgen, dt, dev)
    pt = torch.full((B, mp), pt_fill, dtype=torch.int32)
    if identity:
        for b in range(B):
            pt[b, :n_pages[b]] = torch.arange(b * mp, b * mp + n_pages[b], dtype=torch.int32)
    else:
        perm = torch.randperm(live, generator=gen).to(torch.int32)
        off = 0
        for b in range(B):
            pt[b, :n_pages[b]] = perm[off:off + n_pages[b]]
            off += n_pages[b]
    hot = []
    if hot_tokens:
        for b in range(B):
            pos = torch.randperm(int(ctx[b]), generator=gen)[:hot_tokens]
            hot.append(pos)
            pages = pt[b, (pos // P).long()].long().to(dev)
            slots = (pos % P).to(dev)
            k_cache[pages, :, slots, :] = k_cache[pages, :, slots, :] * hot_scale
    if poison:
        owned = torch.zeros((num_pages, P), dtype=torch.bool)
        for b in range(B):
            T = int(ctx[b])
            for i in range(n_pages[b]):
                owned[int(pt[b, i]), :min(P, T - i * P)] = True
        owned = owned.to(dev)
        nan = torch.tensor(float("nan"), dtype=dt, device=dev)
        k_cache.masked_fill_(~owned[:, None, :, None], nan)
        v_cache.masked_fill_(~owned[:, None, :, None], nan)
    meta = dict(seed=seed, dtype=dtype, identity=identity, pad_pages=pad_pages, hot=hot,
                n_pages=n_pages)
    return DecodeInputs(q, k_cache, v_cache, pt.to(dev), ctx.to(torch.int32).to(dev),
                        1.0 / float(D) ** 0.5, meta)


def prefill_inputs(B, S, Hq, Hkv, D, P, seed=0, *, pad_pages=64, dtype="bf16",
                   device="cpu", cache_fill=float("nan")):
    """Causal prefill inputs: S new tokens per sequence plus a paged pool.

    The pool starts filled with ``cache_fill``; the page table maps the
    ceil(S/P) pages of each sequence through a seeded permutation.
    """
    dt = DTYPES[dtype]
    dev = torch.device(device)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    dgen = gen if dev.type == "cpu" else torch.Generator(device=dev).manual_seed(seed)
    np_ = (S + P - 1) // P
    q = _randn((B, S, Hq, D), dgen, dt, dev)
    k = _randn((B, S, Hkv, D), dgen, dt, dev)
    v = _randn((B, S, Hkv, D), dgen, dt, dev)
    live = B * np_
    perm = torch.randperm(live, generator=gen).to(torch.int32)
    pt = perm.view(B, np_).clone()
    num_pages = live + pad_pages
    k_cache = torch.full((num_pages, Hkv, P, D), cache_fill, dtype=dt, device=dev)
    v_cache = torch.full((num_pages, Hkv, P, D), cache_fill, dtype=dt, device=dev)
    return PrefillInputs(q, k, v, k_cache, v_cache, pt.to(dev), 1.0 / float(D) ** 0.5,
                         dict(seed=seed))


FP8_DTYPES = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}


@dataclass
class Fp8DecodeInputs:
    q: torch.Tensor            # [B][Hq][D] bf16
    k_cache: torch.Tensor      # [num_pages][Hkv][P][D] uint8 (fp8 bytes)
    v_cache: torch.Tensor      # [num_pages][Hkv][P][D] uint8
    k_scale: float             # value of a K byte x = k_scale * fp8(x)
    v_scale: float
    page_table: torch.Tensor   # [B][max_pages] int32
    context_lens: torch.Tensor  # [B] int32
    scale: float
    fmt: str                   # "e4m3" or "e5m2"
    meta: dict = field(default_factory=dict)

    def to(self, device):
        return Fp8DecodeInputs(self.q.to(device), self.k_cache.to(device),
                               self.v_cache.to(device), self.k_scale, self.v_scale,
                               self.page_table.to(device), self.context_lens.to(device),
                               self.scale, self.fmt, dict(self.meta))


def fp8_decode_inputs(B, Hq, Hkv, D, P, lens, fmt="e4m3", seed=0, device="cpu", **kw):
    """Decode inputs with an 8-bit KV pool: the fp32 draw of ``decode_inputs`` (same seed,
    NaN in dead slots), q rounded to bf16, K and V divided by a per-tensor scale that maps
    their largest magnitude to the format's largest finite value and rounded to the format
    by torch (round to nearest even); the pools hold the raw bytes."""
    x = decode_inputs(B, Hq, Hkv, D, P, lens, "f32", seed=seed, device="cpu", **kw)
    ft = FP8_DTYPES[fmt]

    def quant(c):
        amax = float(torch.nan_to_num(c.abs(), nan=0.0).max())
        sc = amax / FP8_MAX[fmt] if amax > 0 else 1.0
        return (c / sc).to(ft).view(torch.uint8), sc

    kq, ks = quant(x.k_cache)
    vq, vs = quant(x.v_cache)
    dev = torch.device(device)
    return Fp8DecodeInputs(x.q.to(torch.bfloat16).to(dev), kq.to(dev), vq.to(dev), ks, vs,
                           x.page_table.to(dev), x.context_lens.to(dev), x.scale, fmt,
                           dict(x.meta, fmt=fmt))


def config2_fp8(fmt="e4m3", device="cpu"):
    """Workload 2 with an 8-bit KV pool: B=64, Hq=32, Hkv=8, D=128, P=16,
    T ~ U{512..4096} (seed 2000, the same lengths and page table)."""
    return fp8_decode_inputs(64, 32, 8, 128, 16, (512, 4096), fmt, seed=2000, device=device)


@dataclass
class ChunkedInputs:
    q: torch.Tensor            # [B][S][Hq][D]: new rows i < new_lens[b] are live
    k: torch.Tensor            # [B][S][Hkv][D]: K of the new tokens
    v: torch.Tensor            # [B][S][Hkv][D]
    k_cache: torch.Tensor      # [num_pages][Hkv][P][D]: the past_lens[b] cached tokens
    v_cache: torch.Tensor
    page_table: torch.Tensor   # [B][max_pages] int32, covers past_lens[b] + new_lens[b]
    past_lens: torch.Tensor    # [B] int32
    new_lens: torch.Tensor     # [B] int32, <= S
    scale: float
    meta: dict = field(default_factory=dict)

    def to(self, device):
        return ChunkedInputs(self.q.to(device), self.k.to(device), self.v.to(device),
                             self.k_cache.to(device), self.v_cache.to(device),
                             self.page_table.to(device), self.past_lens.to(device),
                             self.new_lens.to(device), self.scale, dict(self.meta))


def chunked_inputs(B, S, Hq, Hkv, D, P, past, new=None, seed=0, *, pad_pages=16, dtype="bf16",
                   device="cpu", poison=True):
    """Chunked prefill inputs: sequence b already holds past[b] tokens in the paged pool and
    appends new[b] <= S tokens (default S). ``past`` / ``new``: an int or a list of B ints.

    Draw order: Q, new K, new V, cached K, cached V, page permutation. Pool slots that no
    cached token owns (the tail of the last cached page, the pages of the new tokens, pad
    pages) hold NaN when ``poison``; the page table is padded with -1 past the live pages.
    """
    dt = DTYPES[dtype]
    dev = torch.device(device)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    past = [past] * B if isinstance(past, int) else list(past)
    new = [S] * B if new is None else ([new] * B if isinstance(new, int) else list(new))
    assert len(past) == B and len(new) == B and all(0 <= n <= S for n in new)
    cpu = torch.device("cpu")  # drawn on the host (same values for every device)
    q = _randn((B, S, Hq, D), gen, dt, cpu)
    k = _randn((B, S, Hkv, D), gen, dt, cpu)
    v = _randn((B, S, Hkv, D), gen, dt, cpu)
    n_pages = [(p + n + P - 1) // P for p, n in zip(past, new)]
    max_pages = max(max(n_pages), 1)
    live = sum(n_pages)
    num_pages = live + pad_pages
    fill = float("nan") if poison else 0.0
    k_cache = torch.full((num_pages, Hkv, P, D), fill, dtype=dt)
    v_cache = torch.full((num_pages, Hkv, P, D), fill, dtype=dt)
    kc = [_randn((p, Hkv, D), gen, dt, torch.device("cpu")) for p in past]
    vc = [_randn((p, Hkv, D), gen, dt, torch.device("cpu")) for p in past]
    perm = torch.randperm(live, generator=gen).to(torch.int32)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    o = 0
    for b in range(B):
        pt[b, :n_pages[b]] = perm[o:o + n_pages[b]]
        o += n_pages[b]
        for t in range(past[b]):
            page, slot = int(pt[b, t // P]), t % P
            k_cache[page, :, slot, :] = kc[b][t]
            v_cache[page, :, slot, :] = vc[b][t]
    return ChunkedInputs(q.to(dev), k.to(dev), v.to(dev), k_cache.to(dev), v_cache.to(dev),
                         pt.to(dev),
                         torch.tensor(past, dtype=torch.int32, device=dev),
                         torch.tensor(new, dtype=torch.int32, device=dev),
                         1.0 / float(D) ** 0.5, dict(seed=seed))


# ---- the five workloads ------------------------------------------------------------------

def config1(device="cpu", **kw):
    """Tiny fp32 GQA decode: B=2, Hq=8, Hkv=2, D=64, 256 contiguous tokens each."""
    return decode_inputs(2, 8, 2, 64, 16, 256, "f32", seed=1000, identity=True, pad_pages=0,
                         device=device, **kw)


def config2(device="cpu", **kw):
    """Paged bf16 decode: B=64, Hq=32, Hkv=8, D=128, P=16, T ~ U{512..4096}."""
    return decode_inputs(64, 32, 8, 128, 16, (512, 4096), "bf16", seed=2000, device=device, **kw)


def config3(device="cpu", **kw):
    """Causal bf16 prefill: B=4, S=2048, Hq=32, Hkv=8, D=128, append to P=16 pages."""
    return prefill_inputs(4, 2048, 32, 8, 128, 16, seed=3000, device=device, **kw)


CONFIG4_BATCHES = (1, 4, 8)
CONFIG4_SPLITS = (1, 4, 8, 16)


def config4(B, device="cpu", **kw):
    """Long-context bf16 decode at 32768 tokens with 64 hot keys (x4) per sequence."""
    return decode_inputs(B, 32, 8, 128, 16, 32768, "bf16", seed=4000 + B, hot_tokens=64,
                         device=device, **kw)


CONFIG5_BATCHES = (1, 16, 32, 64, 128, 256)
CONFIG5_KV_HEADS = (1, 8, 32)


def config5(B, Hkv, device="cpu", **kw):
    """Batch/group sweep: Hq=32, T=1024, D=128, P=16, Hkv in {1, 8, 32}."""
    seed = 5000 + 10 * CONFIG5_KV_HEADS.index(Hkv) + CONFIG5_BATCHES.index(B)
    return decode_inputs(B, 32, Hkv, 128, 16, 1024, "bf16", seed=seed, device=device, **kw)
