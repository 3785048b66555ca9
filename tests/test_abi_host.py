"""The C ABI on the host (CPU only): the library loads, exports every symbol the header declares,
and rejects bad arguments with the documented status before anything is launched.

Every call below is built to fail host-side validation (the pointers are fake), so no kernel is
ever launched from this file, with or without a GPU present.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash2.h")
LIB = os.path.join(ROOT, "dflash2_draft_candidate_amd", "libdflash2.so")

OK, EINVAL, EUNSUP, EALIGN, EWS, EHIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
P = 0x100000          # fake, 16-byte aligned, never dereferenced
MIS = 0x100008        # fake, misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__._hip_build_module().build()
    L = ctypes.CDLL(LIB)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.dflash2_select.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, vp] + [ci] * 6 + [vp] * 5 + [sz, vp]
    L.dflash2_select_noalloc.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, vp] + [ci] * 6 + [vp] * 5
    L.dflash2_workspace_bytes.argtypes = [ci] * 6
    L.dflash2_workspace_bytes.restype = sz
    L.dflash2_topk_lse.argtypes = [vp, ci, ci, ci, ci, vp, vp, vp, vp, sz, vp]
    L.dflash2_topk_lse_workspace_bytes.argtypes = [ci] * 4
    L.dflash2_topk_lse_workspace_bytes.restype = sz
    L.dflash2_gate.argtypes = [vp, vp, ci, ci, ci, ci, vp, vp, sz, vp]
    L.dflash2_gate_workspace_bytes.argtypes = [ci] * 3
    L.dflash2_gate_workspace_bytes.restype = sz
    L.dflash2_lattice.argtypes = [vp, vp, vp, vp, vp, ci, vp] + [ci] * 5 + [vp, vp]
    L.dflash2_walk.argtypes = [vp, vp, ci, ci, ci, vp, vp, vp]
    cf = ctypes.c_float
    L.dflash2_walk_ex.argtypes = [vp, vp, ci, ci, ci, cf, vp, cf, vp, vp, vp, vp]
    L.dflash2_select_ex.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, vp] + [ci] * 6 + \
        [cf, vp, cf, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dflash2_dynconv.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, vp, vp]
    L.dflash2_lmhead_topk.argtypes = [vp, vp] + [ci] * 4 + [vp, vp, vp, vp, sz, vp]
    L.dflash2_lmhead_topk_workspace_bytes.argtypes = [ci] * 4
    L.dflash2_lmhead_topk_workspace_bytes.restype = sz
    L.dflash2_status_string.argtypes = [ci]
    L.dflash2_status_string.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash2_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for f in ("dflash2_select", "dflash2_workspace_bytes", "dflash2_status_string",
              "dflash2_topk_lse", "dflash2_gate", "dflash2_lattice", "dflash2_walk",
              "dflash2_select_ex", "dflash2_walk_ex", "dflash2_dynconv", "dflash2_lmhead_topk",
              "dflash2_select_noalloc",
              "dflash2_lmhead_topk_workspace_bytes"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_covers_the_abi():
    import dflash2_draft_candidate_amd as d2
    assert sorted(d2.EXPORTS) == declared_functions()
    assert d2.version() == 3


def test_status_strings(lib):
    for s in (OK, EINVAL, EUNSUP, EALIGN, EWS, EHIP, 12345):
        assert lib.dflash2_status_string(s)


def sel(lib, *, logits=P, ld=BF16, hidden=P, ad=BF16, W=P, pred=P, succ=P, cd=BF16, anchor=P,
        B=2, L=4, V=1000, H=64, r=16, k=8, cand=P, unary=P, edges=P, path=P, ws=P, wsb=None):
    if wsb is None:
        wsb = 0  # too small unless a test passes a size: such calls stop at the workspace check
    return lib.dflash2_select(logits, ld, hidden, ad, W, pred, succ, cd, anchor, B, L, V, H, r, k,
                              cand, unary, edges, path, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), EINVAL), (dict(k=65), EINVAL), (dict(k=9, V=8), EINVAL), (dict(B=0), EINVAL),
    (dict(L=0), EINVAL), (dict(V=0), EINVAL), (dict(H=0), EINVAL), (dict(r=0), EINVAL),
    (dict(r=257), EINVAL), (dict(ld=2), EINVAL), (dict(ad=-1), EINVAL), (dict(cd=5), EINVAL),
    (dict(logits=None), EINVAL), (dict(anchor=None), EINVAL), (dict(path=None), EINVAL),
    (dict(hidden=MIS), EALIGN), (dict(edges=MIS), EALIGN), (dict(ws=None), EWS),
    (dict(), EWS),                        # workspace size 0 < required
    (dict(ws=MIS, wsb=1 << 30), EALIGN),
])
def test_select_rejects(lib, kw, status):
    assert sel(lib, **kw) == status


def test_workspace_sizes(lib):
    assert lib.dflash2_workspace_bytes(0, 4, 1000, 64, 16, 8) == 0
    assert lib.dflash2_workspace_bytes(1, 4, 1000, 64, 16, 65) == 0
    small = lib.dflash2_workspace_bytes(1, 16, 151936, 4096, 64, 16)
    big = lib.dflash2_workspace_bytes(64, 16, 151936, 4096, 64, 16)
    assert small > 0 and big > 0
    # lse and g alone need R * (1 + r) floats
    assert big >= 1024 * 65 * 4
    assert lib.dflash2_topk_lse_workspace_bytes(16, 151936, 16, BF16) > 0   # sliced rows
    assert lib.dflash2_topk_lse_workspace_bytes(2048, 151936, 32, F32) == 0  # one slice per row
    assert lib.dflash2_topk_lse_workspace_bytes(4, 100, 101, F32) == 0      # invalid k


def test_stage_entry_points_reject(lib):
    assert lib.dflash2_topk_lse(P, F32, 4, 100, 0, P, P, P, P, 1 << 20, None) == EINVAL
    assert lib.dflash2_topk_lse(P, 3, 4, 100, 4, P, P, P, P, 1 << 20, None) == EINVAL
    assert lib.dflash2_topk_lse(P, F32, 4, 100, 4, MIS, P, P, P, 1 << 20, None) == EALIGN
    assert lib.dflash2_topk_lse(P, BF16, 16, 151936, 16, P, P, P, None, 0, None) == EWS
    assert lib.dflash2_gate(P, P, F32, 4, 64, 300, P, P, 0, None) == EINVAL
    assert lib.dflash2_gate(None, P, F32, 4, 64, 16, P, P, 0, None) == EINVAL
    assert lib.dflash2_gate(P, P, BF16, 1024, 4096, 64, P, None, 0, None) == EWS
    assert lib.dflash2_lattice(P, P, P, P, P, F32, P, 2, 3, 100, 16, 65, P, None) == EINVAL
    assert lib.dflash2_lattice(P, P, P, P, MIS, F32, P, 2, 3, 100, 16, 4, P, None) == EALIGN
    assert lib.dflash2_walk(P, P, 2, 3, 0, P, P, None) == EINVAL
    assert lib.dflash2_walk(P, P, 2, 3, 4, P, MIS, None) == EALIGN
    assert lib.dflash2_walk(None, P, 2, 3, 4, P, None, None) == EINVAL


def test_mode_entry_points_reject(lib):
    nan, inf = float("nan"), float("inf")
    # walk_ex: sizes, temperature (negative, NaN, infinite), p_min NaN, sampling without
    # uniforms, misaligned optional outputs
    assert lib.dflash2_walk_ex(P, P, 2, 3, 0, 0.0, None, 0.0, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, -1.0, None, 0.0, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, nan, None, 0.0, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, inf, P, 0.0, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, 0.0, None, nan, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, 1.0, None, 0.0, P, None, None, None) == EINVAL
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, 1.0, MIS, 0.0, P, None, None, None) == EALIGN
    assert lib.dflash2_walk_ex(P, P, 2, 3, 4, 0.0, None, 0.5, P, None, MIS, None) == EALIGN
    assert lib.dflash2_walk_ex(None, P, 2, 3, 4, 0.0, None, 0.0, P, None, None, None) == EINVAL

    def sx(T=0.0, u=None, p_min=0.0, dlen=None, k=8, wsb=1 << 30):
        return lib.dflash2_select_ex(P, BF16, P, BF16, P, P, P, BF16, P, 2, 4, 1000, 64, 16, k,
                                     T, u, p_min, P, P, P, P, dlen, P, wsb, None)
    assert sx(k=0) == EINVAL
    assert sx(T=-0.5) == EINVAL
    assert sx(T=nan) == EINVAL
    assert sx(T=1.0) == EINVAL            # sampling needs uniforms
    assert sx(p_min=nan) == EINVAL
    assert sx(T=1.0, u=MIS) == EALIGN
    assert sx(dlen=MIS) == EALIGN


@pytest.mark.parametrize("kw,status", [
    (dict(K=0), EINVAL), (dict(K=9), EINVAL), (dict(G=0), EINVAL), (dict(G=5), EINVAL),
    (dict(nb=0), EINVAL), (dict(T=0), EINVAL), (dict(C=0), EINVAL), (dict(dt=2), EINVAL),
    (dict(x=None), EINVAL), (dict(y=None), EINVAL), (dict(dyn=MIS), EALIGN), (dict(y=MIS), EALIGN),
])
def test_dynconv_rejects(lib, kw, status):
    a = dict(x=P, base=P, dyn=P, dt=BF16, nb=2, T=5, C=64, K=2, G=16, y=P)
    a.update(kw)
    assert lib.dflash2_dynconv(a["x"], a["base"], a["dyn"], a["dt"], a["nb"], a["T"], a["C"],
                               a["K"], a["G"], a["y"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), EINVAL), (dict(k=17), EINVAL), (dict(k=101), EINVAL), (dict(H=12), EINVAL),
    (dict(H=0), EINVAL), (dict(R=0), EINVAL), (dict(V=0), EINVAL), (dict(hidden=None), EINVAL),
    (dict(W=None), EINVAL), (dict(ids=None), EINVAL), (dict(W=MIS), EALIGN),
    (dict(lse=MIS), EALIGN), (dict(ws=None), EWS), (dict(wsb=16), EWS), (dict(ws=MIS), EALIGN),
    # more than one 16-row tile: refused (a library product and the top-k pass are faster there)
    (dict(R=17), EUNSUP), (dict(R=1024), EUNSUP), (dict(R=17, k=0), EINVAL),
])
def test_lmhead_rejects(lib, kw, status):
    a = dict(hidden=P, W=P, R=16, H=64, V=100, k=16, ids=P, un=P, lse=None, ws=P, wsb=1 << 30)
    a.update(kw)
    assert lib.dflash2_lmhead_topk(a["hidden"], a["W"], a["R"], a["H"], a["V"], a["k"], a["ids"],
                                   a["un"], a["lse"], a["ws"], a["wsb"], None) == status


def test_lmhead_workspace_sizes(lib):
    assert lib.dflash2_lmhead_topk_workspace_bytes(16, 4096, 151936, 16) > 0
    assert lib.dflash2_lmhead_topk_workspace_bytes(16, 4096, 151936, 17) == 0
    assert lib.dflash2_lmhead_topk_workspace_bytes(16, 4100, 151936, 16) == 0
    assert lib.dflash2_lmhead_topk_workspace_bytes(17, 4096, 151936, 16) == 0


def test_binding_rejects_host_tensors():
    import torch
    import dflash2_draft_candidate_amd as d2
    with pytest.raises(ValueError):
        d2.topk_lse(torch.zeros(2, 10), 2)


def _noalloc(lib, B=2, L=4, V=1000, H=64, r=16, k=8, ptrs=None, dts=(BF16, BF16, BF16)):
    p = ptrs or {}
    g = lambda n: p.get(n, P)
    return lib.dflash2_select_noalloc(g("logits"), dts[0], g("hidden"), dts[1], g("W"), g("pred"),
                                      g("succ"), dts[2], g("anchor"), B, L, V, H, r, k,
                                      g("ids"), g("unary"), g("edges"), g("path"), None)


def test_select_noalloc_validation(lib):
    # the same argument errors as dflash2_select, all before the scratch array is looked up
    assert _noalloc(lib, k=0) == EINVAL
    assert _noalloc(lib, k=65) == EINVAL
    assert _noalloc(lib, r=257) == EINVAL
    assert _noalloc(lib, V=4, k=8) == EINVAL
    assert _noalloc(lib, dts=(BF16, 7, BF16)) == EINVAL
    assert _noalloc(lib, ptrs={"edges": None}) == EINVAL
    assert _noalloc(lib, ptrs={"hidden": MIS}) == EALIGN


def test_select_noalloc_size_limit(lib):
    # more than DFLASH2_NOALLOC_SCRATCH_BYTES of workspace: refused before anything runs
    limit = 16 << 20
    big = (2048, 16, 262144, 8192, 256, 64)
    assert lib.dflash2_workspace_bytes(*big) > limit
    B, L, V, H, r, k = big
    assert _noalloc(lib, B, L, V, H, r, k) == EWS
    serving = (64, 16, 151936, 4096, 64, 16)
    assert lib.dflash2_workspace_bytes(*serving) <= limit
