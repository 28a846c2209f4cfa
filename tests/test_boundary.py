"""C-ABI boundary tests that need no GPU.

The library must load, export every function that include/gqa.h declares, and
reject invalid arguments on the host with the documented status codes before
anything is enqueued (so these calls never touch a device).
"""

import ctypes
import os
import re

import pytest

import gqa_paged_kv_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gqa.h", "gqa_bench.h")]
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(g.LIB_PATH):
        from gqa_paged_kv_amd import build
        build.build()
    return g.load()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("gqa_decode_paged", "gqa_prefill_causal", "gqa_combine_splits"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(g.SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings(lib):
    assert g.status_string(0) == "ok"
    assert "invalid" in g.status_string(1)
    assert "unsupported" in g.status_string(2)
    assert "launch" in g.status_string(3)
    assert "scratch" in g.status_string(4)


def test_workspace_bytes(lib):
    assert g.workspace_bytes(8, 32, 128, 16) == 8 * 32 * 16 * (128 + 1) * 4
    assert g.workspace_bytes(0, 32, 128, 16) == 0


def test_balanced_workspace_layout(lib):
    """The counter region the header reserves at the start of a balanced-decode workspace is
    the one the binding knows, and the size function adds it to the larger of the persistent
    path's slots (whole 128-byte lines per piece) and the split path's partials."""
    text = open(os.path.join(ROOT, "include", "gqa.h")).read()
    m = re.search(r"#define\s+GQA_BALANCED_WS_RESERVED\s+(\d+)", text)
    assert m and int(m.group(1)) == g.BALANCED_WS_RESERVED == 3 * 4096 * 8  # 64-bit counters
    n = lib.gqa_decode_balanced_workspace_bytes
    slot_floats = (4 * 128 + 4 + 31) // 32 * 32  # G = 4, D = 128
    assert n(64, 32, 8, 128) == g.BALANCED_WS_RESERVED + 4096 * 2 * slot_floats * 4
    assert n(64, 32, 8, 128) % 256 == 0
    assert n(0, 32, 8, 128) == 0 and n(4, 30, 8, 128) == 0
    # G >= 16 takes the split path: counters, then its partials only
    assert n(8, 32, 1, 128) == g.BALANCED_WS_RESERVED + g.workspace_bytes(8, 32, 128, 16)  # NS = 16
    assert n(256, 32, 1, 128) == g.BALANCED_WS_RESERVED  # one split: no partials


def test_balanced_route_limits(lib):
    """The balanced entry point's route: the split path (n >= 1 splits) at or below 1,024
    (sequence, KV head, page) items (65,536 for G = 1), and for G = 2 / G = 4 at or below
    16,384 / 8,192 items when it takes at most 4 splits of rows of at least 16 pages; the
    persistent kernel (0) otherwise; the split path for G >= 16 at every size, and the
    persistent kernel whenever the split partials would not fit in the workspace."""
    r = g.balanced_route
    # G = 4: B * Hkv * max_pages = 1024 / 1032 with 8 splits
    assert r(2, 32, 8, 128, 64) >= 1 and r(2, 32, 8, 128, 64) == min(256 // 16, 64 // 16)
    assert r(1, 32, 8, 128, 128) >= 1 and r(1, 32, 8, 128, 129) == 0
    assert r(2, 32, 8, 128, 128) == 0  # 2,048 items, 8 splits
    # G = 4, at most 4 splits of 16+ page rows: 8192 / 8256 items
    assert r(5, 20, 5, 128, 41) == 2 and r(5, 20, 5, 128, 40) >= 1  # 1025 / 1000 items
    assert r(8, 32, 8, 128, 128) == 4 and r(8, 32, 8, 128, 129) == 0
    assert r(64, 32, 8, 128, 8) == 0 and r(64, 32, 8, 128, 16) == 1  # 8-page rows
    # G = 1: 65536 / 65537 items
    assert r(8, 8, 8, 128, 1024) >= 1 and r(8, 8, 8, 128, 1025) == 0
    assert r(1, 1, 1, 128, 65536) >= 1 and r(1, 1, 1, 128, 65537) == 0
    # G = 8 follows the 1,024 rule; G = 2 the 16,384 one (16384 / 16512 items)
    assert r(4, 32, 4, 64, 64) >= 1 and r(4, 32, 4, 64, 65) == 0
    assert r(1, 32, 16, 128, 64) >= 1 and r(1, 32, 16, 128, 65) == 4
    assert r(8, 32, 16, 128, 128) == 2 and r(8, 32, 16, 128, 129) == 0
    # narrow tables: at least 16 pages per split, so fewer than 32 pages means one split
    assert r(2, 8, 2, 128, 16) == 1 and r(2, 8, 2, 128, 31) == 1 and r(2, 8, 2, 128, 32) == 2
    # a workspace that holds only the counters keeps small problems on the persistent kernel
    assert r(2, 32, 8, 128, 64, g.BALANCED_WS_RESERVED) == 0
    # G >= 16: always the split path, one workgroup per CU (at most 16 splits) and at least 8
    # pages per split
    for B, hkv, ns in ((1, 1, 16), (8, 1, 16), (32, 1, 8), (64, 1, 4), (256, 1, 1), (64, 2, 2)):
        assert r(B, 32, hkv, 128, 100000) == ns, (B, hkv)
        assert r(B, 32, hkv, 128, 64) == min(ns, 64 // 8), (B, hkv)
        assert r(B, 32, hkv, 128, 16) == min(ns, 2), (B, hkv)
    assert r(1, 32, 1, 128, 7) == 1 and r(1, 32, 1, 128, 8) == 1 and r(1, 32, 1, 128, 24) == 3
    assert r(0, 32, 8, 128, 64) == -1 and r(2, 30, 8, 128, 64) == -1


def test_page_table_check(lib):
    """gqa_check_page_table: every page id a call touches must lie in [0, num_pages); entries
    past ceil(tokens / P) are never looked at; tokens are clamped to the row width."""
    import torch
    pt = torch.tensor([[3, 0, -1, 99], [1, 2, 5, 7]], dtype=torch.int32)
    chk = lambda tok, n=8: g.check_page_table(pt, torch.tensor(tok, dtype=torch.int32), n)
    assert chk([32, 64]) == g.OK            # row 0: pages 3, 0; row 1: all four < 8
    assert chk([33, 64]) == g.ERR_INVALID_ARG  # row 0 reaches the -1 entry
    assert chk([0, 48]) == g.OK
    assert chk([-5, 48]) == g.OK            # negative lengths touch nothing
    assert chk([32, 64], n=7) == g.ERR_INVALID_ARG  # page 7 outside a 7-page pool
    assert chk([32, 10**6], n=8) == g.OK    # clamped to max_pages * P = 64
    assert chk([10**6, 0]) == g.ERR_INVALID_ARG  # clamped: row 0 reaches -1 and 99
    pt[0, 2], pt[0, 3] = 4, 8
    assert chk([64, 0]) == g.ERR_INVALID_ARG  # 8 == num_pages is outside
    assert chk([64, 0], n=9) == g.OK
    assert lib.gqa_check_page_table(None, None, 2, 4, 16, 8) == g.ERR_INVALID_ARG


def _vd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, pt=FAKE, lens=FAKE, out=FAKE, wo=None, wl=None, B=2, Hq=8,
             Hkv=2, D=128, P=16, max_pages=4, num_pages=8, ns=1, scale=0.125, dtype=g.BF16)
    a.update(kw)
    return lib.gqa_validate_decode(a["q"], a["k"], a["v"], a["pt"], a["lens"], a["out"], a["wo"],
                                   a["wl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["P"],
                                   a["max_pages"], a["num_pages"], a["ns"], a["scale"], a["dtype"])


def test_decode_validation_rules(lib):
    assert _vd(lib) == g.OK
    assert _vd(lib, dtype=g.F32, D=64) == g.OK
    for G in (1, 2, 4, 8, 16, 32):
        assert _vd(lib, Hq=32, Hkv=32 // G) == g.OK
    # invalid arguments
    assert _vd(lib, Hq=6, Hkv=4) == g.ERR_INVALID_ARG  # non-uniform grouping
    for k in ("B", "Hq", "Hkv", "D", "P", "max_pages", "num_pages"):
        assert _vd(lib, **{k: 0}) == g.ERR_INVALID_ARG, k
        assert _vd(lib, **{k: -3}) == g.ERR_INVALID_ARG, k
    for k in ("q", "k", "v", "pt", "lens", "out"):
        assert _vd(lib, **{k: None}) == g.ERR_INVALID_ARG, k
    assert _vd(lib, ns=0) == g.ERR_INVALID_ARG
    assert _vd(lib, ns=4) == g.ERR_INVALID_ARG  # NS > 1 without workspace
    assert _vd(lib, ns=4, wo=FAKE, wl=FAKE) == g.OK
    assert _vd(lib, ns=4, wo=FAKE) == g.ERR_INVALID_ARG
    assert _vd(lib, scale=float("nan")) == g.ERR_INVALID_ARG
    assert _vd(lib, scale=float("inf")) == g.ERR_INVALID_ARG
    assert _vd(lib, dtype=7) == g.ERR_INVALID_ARG
    # valid but not built
    assert _vd(lib, D=96) == g.ERR_UNSUPPORTED
    assert _vd(lib, P=32) == g.ERR_UNSUPPORTED
    assert _vd(lib, Hq=48, Hkv=1) == g.ERR_UNSUPPORTED  # G = 48
    assert _vd(lib, Hq=12, Hkv=4) == g.ERR_UNSUPPORTED  # G = 3
    assert _vd(lib, ns=1000, wo=FAKE, wl=FAKE) == g.ERR_UNSUPPORTED


def _vp(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, out=FAKE, B=4, S=2048, Hq=32,
             Hkv=8, D=128, P=16, max_pages=128, num_pages=600, scale=0.088, dtype=g.BF16)
    a.update(kw)
    return lib.gqa_validate_prefill(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"], a["out"],
                                    a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["P"],
                                    a["max_pages"], a["num_pages"], a["scale"], a["dtype"])


def test_prefill_validation_rules(lib):
    assert _vp(lib) == g.OK
    assert _vp(lib, max_pages=127) == g.ERR_INVALID_ARG  # max_pages * P < S
    assert _vp(lib, S=0) == g.ERR_INVALID_ARG
    assert _vp(lib, Hq=30) == g.ERR_INVALID_ARG
    for k in ("q", "k", "v", "kc", "vc", "pt", "out"):
        assert _vp(lib, **{k: None}) == g.ERR_INVALID_ARG, k
    assert _vp(lib, dtype=g.F32) == g.ERR_UNSUPPORTED
    assert _vp(lib, Hq=32, Hkv=2) == g.ERR_UNSUPPORTED  # G = 16 not built for prefill
    assert _vp(lib, D=64) == g.ERR_UNSUPPORTED
    assert _vp(lib, P=8) == g.ERR_UNSUPPORTED


def _vpp(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, pt=FAKE, past=FAKE, new=FAKE, out=FAKE,
             B=4, S=512, Hq=32, Hkv=8, D=128, P=16, max_pages=8, num_pages=512, scale=0.088,
             dtype=g.BF16)
    a.update(kw)
    return lib.gqa_validate_prefill_paged(a["q"], a["k"], a["v"], a["kc"], a["vc"], a["pt"],
                                          a["past"], a["new"], a["out"], a["B"], a["S"], a["Hq"],
                                          a["Hkv"], a["D"], a["P"], a["max_pages"],
                                          a["num_pages"], a["scale"], a["dtype"])


def test_chunked_prefill_validation_rules(lib):
    assert _vpp(lib) == g.OK  # max_pages * P < S is allowed: lengths are clamped on device
    for k in ("q", "k", "v", "kc", "vc", "pt", "past", "new", "out"):
        assert _vpp(lib, **{k: None}) == g.ERR_INVALID_ARG, k
    assert _vpp(lib, S=0) == g.ERR_INVALID_ARG
    assert _vpp(lib, Hq=30) == g.ERR_INVALID_ARG
    assert _vpp(lib, dtype=g.F32) == g.ERR_UNSUPPORTED
    assert _vpp(lib, Hq=32, Hkv=1) == g.ERR_UNSUPPORTED  # G = 32 not built for prefill
    assert _vpp(lib, D=64) == g.ERR_UNSUPPORTED
    assert _vpp(lib, P=32) == g.ERR_UNSUPPORTED


def test_fp8_decode_validation_rules(lib):
    v = lib.gqa_validate_decode_fp8
    args = lambda **kw: dict(dict(q=FAKE, k=FAKE, vv=FAKE, ks=0.01, vs=0.02, pt=FAKE, lens=FAKE,
                                  out=FAKE, B=4, Hq=32, Hkv=8, D=128, P=16, mp=64, npg=4096,
                                  scale=0.088, dt=g.FP8_E4M3), **kw)
    call = lambda a: v(a["q"], a["k"], a["vv"], a["ks"], a["vs"], a["pt"], a["lens"], a["out"],
                       a["B"], a["Hq"], a["Hkv"], a["D"], a["P"], a["mp"], a["npg"], a["scale"],
                       a["dt"])
    assert call(args()) == g.OK
    assert call(args(dt=g.FP8_E5M2)) == g.OK
    for bad in (dict(dt=g.BF16), dict(dt=7), dict(ks=0.0), dict(vs=-1.0), dict(ks=float("inf")),
                dict(k=None), dict(lens=None), dict(Hq=30)):
        assert call(args(**bad)) == g.ERR_INVALID_ARG, bad
    assert call(args(D=64)) == g.ERR_UNSUPPORTED
    assert call(args(Hq=32, Hkv=2)) == g.ERR_UNSUPPORTED  # G = 16: not built for 8-bit caches


def test_combine_validation_rules(lib):
    v = lib.gqa_validate_combine
    assert v(FAKE, FAKE, FAKE, 4, 32, 128, 8, g.BF16) == g.OK
    assert v(None, FAKE, FAKE, 4, 32, 128, 8, g.BF16) == g.ERR_INVALID_ARG
    assert v(FAKE, FAKE, FAKE, 4, 32, 128, 0, g.BF16) == g.ERR_INVALID_ARG
    assert v(FAKE, FAKE, FAKE, 4, 32, 100, 8, g.BF16) == g.ERR_UNSUPPORTED
    assert v(FAKE, FAKE, FAKE, 4, 32, 128, 8, 5) == g.ERR_INVALID_ARG


def test_entry_points_reject_before_enqueueing(lib):
    # Invalid calls return their status without touching the device.
    st = lib.gqa_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 2, 6, 4, 128, 16,
                              4, 8, 1, 0.1, g.BF16, None)
    assert st == g.ERR_INVALID_ARG
    st = lib.gqa_prefill_causal(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 8, 2, 128, 16,
                                4, 8, 0.1, g.F32, None)
    assert st == g.ERR_UNSUPPORTED
    st = lib.gqa_prefill_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 64, 8,
                               2, 128, 16, 4, 8, 0.1, g.BF16, None)
    assert st == g.ERR_INVALID_ARG
    st = lib.gqa_decode_paged_fp8(FAKE, FAKE, FAKE, 0.0, 1.0, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2,
                                  8, 2, 128, 16, 4, 8, 0.1, g.FP8_E4M3, None)
    assert st == g.ERR_INVALID_ARG
    st = lib.gqa_decode_append(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2,
                               8, 2, 128, 16, 4, 8, 0.1, g.BF16, None)
    assert st == g.ERR_INVALID_ARG
    st = lib.gqa_decode_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 2,
                               32, 2, 128, 16, 4, 8, 0.1, g.BF16, None)
    assert st == g.ERR_UNSUPPORTED  # G = 16
    st = lib.gqa_combine_splits(FAKE, None, FAKE, 1, 8, 128, 2, g.BF16, None)
    assert st == g.ERR_INVALID_ARG
    st = lib.gqa_gather_paged(FAKE, FAKE, FAKE, FAKE, 1, 2, 96, 16, 4, 8, g.BF16, None)
    assert st == g.ERR_UNSUPPORTED


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "gqa_paged_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "oracle" not in text.lower().replace("oracles", ""), f
