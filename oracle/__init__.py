"""Oracle for the DFlash 2 candidate-selector lattice (plain fp64 C, loaded through ctypes).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product library (``dflash2_draft_candidate_amd``) never
imports it, and it never imports the product library.

The arithmetic lives in ``dflash2_oracle.c``; this module only compiles it (gcc, no HIP) and
marshals numpy arrays. Stored tensors are numpy ``float32`` for fp32 and ``uint16`` (raw bits)
for bf16. Outputs are float64 (scores) and int32 (ids).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dflash2_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

F32 = 0
BF16 = 1

_c_int_p = ctypes.POINTER(ctypes.c_int32)
_c_dbl_p = ctypes.POINTER(ctypes.c_double)


def compile_oracle(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc into a shared library (IEEE double, no contraction)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"stored tensors are float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class SelectResult:
    cand_ids: np.ndarray  # [B, L, k] int32
    unary: np.ndarray     # [B, L, k] float64
    edges: np.ndarray     # [B, L, k, k] float64
    path: np.ndarray      # [B, L] int32
    lse: np.ndarray       # [B, L] float64
    path_idx: np.ndarray  # [B, L] int32
    margin: np.ndarray    # [B, L] float64
    score: np.ndarray     # [B] float64


class Oracle:
    """ctypes view of one compiled oracle library (the default one, or another build of it)."""

    def __init__(self, lib_path: str = LIBRARY):
        if not os.path.exists(lib_path):
            compile_oracle(SOURCE, lib_path)
        self.lib = ctypes.CDLL(lib_path)
        vp, ci = ctypes.c_void_p, ctypes.c_int
        self.lib.dflash2_ref_topk_lse.argtypes = [vp, ci, ci, ci, ci, _c_int_p, _c_dbl_p, _c_dbl_p]
        self.lib.dflash2_ref_gate.argtypes = [vp, vp, ci, ci, ci, ci, _c_dbl_p]
        self.lib.dflash2_ref_lattice.argtypes = [_c_int_p, _c_dbl_p, _c_dbl_p, vp, vp, ci, _c_int_p,
                                                 ci, ci, ci, ci, ci, _c_dbl_p]
        self.lib.dflash2_ref_walk.argtypes = [_c_dbl_p, _c_int_p, ci, ci, ci, _c_int_p, _c_int_p,
                                              _c_dbl_p, _c_dbl_p]
        self.lib.dflash2_ref_walk_ex.argtypes = [_c_dbl_p, _c_int_p, ci, ci, ci, ctypes.c_double,
                                                 _c_dbl_p, ctypes.c_double, _c_int_p, _c_int_p,
                                                 _c_int_p, _c_dbl_p, _c_dbl_p]
        self.lib.dflash2_ref_dynconv.argtypes = [vp, vp, vp, ci, ci, ci, ci, ci, ci, _c_dbl_p]
        self.lib.dflash2_ref_lmhead_topk.argtypes = [vp, vp, ci, ci, ci, ci, ci, _c_int_p, _c_dbl_p,
                                                     _c_dbl_p, _c_dbl_p]
        self.lib.dflash2_ref_select.argtypes = [vp, ci, vp, ci, vp, vp, vp, ci, _c_int_p, ci, ci, ci,
                                                ci, ci, ci, _c_int_p, _c_dbl_p, _c_dbl_p, _c_int_p,
                                                _c_dbl_p, _c_int_p, _c_dbl_p, _c_dbl_p]
        for f in ("dflash2_ref_topk_lse", "dflash2_ref_gate", "dflash2_ref_lattice",
                  "dflash2_ref_walk", "dflash2_ref_select", "dflash2_ref_lmhead_topk"):
            getattr(self.lib, f).restype = ctypes.c_int

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")

    def topk_lse(self, logits: np.ndarray, k: int):
        """logits [R, V] (float32 or bf16 bits) -> cand_ids [R,k] int32, unary [R,k], lse [R]."""
        logits = np.ascontiguousarray(logits)
        R, V = logits.shape
        ids = np.zeros((R, k), np.int32)
        unary = np.zeros((R, k), np.float64)
        lse = np.zeros((R,), np.float64)
        rc = self.lib.dflash2_ref_topk_lse(_ptr(logits), dtype_code(logits), R, V, k,
                                           ids.ctypes.data_as(_c_int_p),
                                           unary.ctypes.data_as(_c_dbl_p),
                                           lse.ctypes.data_as(_c_dbl_p))
        self._check(rc, "topk_lse")
        return ids, unary, lse

    def lmhead_topk(self, hidden: np.ndarray, W_lm: np.ndarray, k: int, want_logits=False):
        """hidden [R, H], W_lm [V, H] (same dtype) -> cand_ids [R,k] int32, unary [R,k], lse [R]
        (and the logits [R, V] float64 when want_logits)."""
        hidden = np.ascontiguousarray(hidden)
        W_lm = np.ascontiguousarray(W_lm)
        if hidden.dtype != W_lm.dtype:
            raise TypeError("hidden and W_lm share one dtype")
        R, H = hidden.shape
        V, H2 = W_lm.shape
        if H2 != H:
            raise ValueError("W_lm must be [V, H]")
        ids = np.zeros((R, k), np.int32)
        unary = np.zeros((R, k), np.float64)
        lse = np.zeros((R,), np.float64)
        x = np.zeros((R, V), np.float64) if want_logits else None
        rc = self.lib.dflash2_ref_lmhead_topk(
            _ptr(hidden), _ptr(W_lm), dtype_code(hidden), R, H, V, k,
            ids.ctypes.data_as(_c_int_p), unary.ctypes.data_as(_c_dbl_p),
            lse.ctypes.data_as(_c_dbl_p), None if x is None else x.ctypes.data_as(_c_dbl_p))
        self._check(rc, "lmhead_topk")
        return (ids, unary, lse, x) if want_logits else (ids, unary, lse)

    def gate(self, hidden: np.ndarray, W_sel: np.ndarray):
        """hidden [R, H], W_sel [H, r] (same dtype) -> g [R, r] float64."""
        hidden = np.ascontiguousarray(hidden)
        W_sel = np.ascontiguousarray(W_sel)
        if hidden.dtype != W_sel.dtype:
            raise TypeError("hidden and W_sel share one dtype")
        R, H = hidden.shape
        H2, r = W_sel.shape
        if H2 != H:
            raise ValueError("W_sel must be [H, r]")
        g = np.zeros((R, r), np.float64)
        rc = self.lib.dflash2_ref_gate(_ptr(hidden), _ptr(W_sel), dtype_code(hidden), R, H, r,
                                       g.ctypes.data_as(_c_dbl_p))
        self._check(rc, "gate")
        return g

    def lattice(self, cand_ids, unary, g, pred_cb, succ_cb, anchor_ids):
        """cand_ids/unary [B,L,k], g [B,L,r] float64, codebooks [V,r], anchor_ids [B] -> edges."""
        cand_ids = np.ascontiguousarray(cand_ids, dtype=np.int32)
        unary = np.ascontiguousarray(unary, dtype=np.float64)
        g = np.ascontiguousarray(g, dtype=np.float64)
        pred_cb = np.ascontiguousarray(pred_cb)
        succ_cb = np.ascontiguousarray(succ_cb)
        anchor_ids = np.ascontiguousarray(anchor_ids, dtype=np.int32)
        if pred_cb.dtype != succ_cb.dtype or pred_cb.shape != succ_cb.shape:
            raise TypeError("pred_cb and succ_cb share one dtype and shape")
        B, L, k = cand_ids.shape
        V, r = pred_cb.shape
        edges = np.zeros((B, L, k, k), np.float64)
        rc = self.lib.dflash2_ref_lattice(cand_ids.ctypes.data_as(_c_int_p),
                                          unary.ctypes.data_as(_c_dbl_p),
                                          g.ctypes.data_as(_c_dbl_p), _ptr(pred_cb), _ptr(succ_cb),
                                          dtype_code(pred_cb), anchor_ids.ctypes.data_as(_c_int_p),
                                          B, L, V, r, k, edges.ctypes.data_as(_c_dbl_p))
        self._check(rc, "lattice")
        return edges

    def walk(self, edges, cand_ids):
        """edges [B,L,k,k] (any float; read as float64), cand_ids [B,L,k] -> path, idx, margin, score."""
        edges = np.ascontiguousarray(edges, dtype=np.float64)
        cand_ids = np.ascontiguousarray(cand_ids, dtype=np.int32)
        B, L, k = cand_ids.shape
        path = np.zeros((B, L), np.int32)
        idx = np.zeros((B, L), np.int32)
        margin = np.zeros((B, L), np.float64)
        score = np.zeros((B,), np.float64)
        rc = self.lib.dflash2_ref_walk(edges.ctypes.data_as(_c_dbl_p),
                                       cand_ids.ctypes.data_as(_c_int_p), B, L, k,
                                       path.ctypes.data_as(_c_int_p), idx.ctypes.data_as(_c_int_p),
                                       margin.ctypes.data_as(_c_dbl_p),
                                       score.ctypes.data_as(_c_dbl_p))
        self._check(rc, "walk")
        return path, idx, margin, score

    def walk_ex(self, edges, cand_ids, temperature: float = 0.0, uniforms=None,
                p_min: float = 0.0):
        """The walk with sampling at temperature T (uniforms [B,L] in [0,1)) and the p_min early
        stop -> path, idx, draft_len [B], conf [B,L], cdf_margin [B,L]."""
        edges = np.ascontiguousarray(edges, dtype=np.float64)
        cand_ids = np.ascontiguousarray(cand_ids, dtype=np.int32)
        B, L, k = cand_ids.shape
        u = None if uniforms is None else np.ascontiguousarray(uniforms, dtype=np.float64)
        path = np.zeros((B, L), np.int32)
        idx = np.zeros((B, L), np.int32)
        dlen = np.zeros((B,), np.int32)
        conf = np.zeros((B, L), np.float64)
        cm = np.zeros((B, L), np.float64)
        rc = self.lib.dflash2_ref_walk_ex(
            edges.ctypes.data_as(_c_dbl_p), cand_ids.ctypes.data_as(_c_int_p), B, L, k,
            float(temperature), None if u is None else u.ctypes.data_as(_c_dbl_p), float(p_min),
            path.ctypes.data_as(_c_int_p), idx.ctypes.data_as(_c_int_p),
            dlen.ctypes.data_as(_c_int_p), conf.ctypes.data_as(_c_dbl_p),
            cm.ctypes.data_as(_c_dbl_p))
        self._check(rc, "walk_ex")
        return path, idx, dlen, conf, cm

    def dynconv(self, x, base, dyn, group: int):
        """x [nb,T,C], base [K,C], dyn [nb,T,K,C/group] (one stored dtype) -> y [nb,T,C] float64."""
        x = np.ascontiguousarray(x)
        base = np.ascontiguousarray(base)
        dyn = np.ascontiguousarray(dyn)
        nb, T, C = x.shape
        K = base.shape[0]
        dt = dtype_code(x)
        if dtype_code(base) != dt or dtype_code(dyn) != dt:
            raise ValueError("x, base and dyn must share a stored dtype")
        if base.shape != (K, C) or dyn.shape != (nb, T, K, C // group):
            raise ValueError("inconsistent shapes")
        y = np.zeros((nb, T, C), np.float64)
        rc = self.lib.dflash2_ref_dynconv(_ptr(x), _ptr(base), _ptr(dyn), dt, nb, T, C, K, group,
                                          y.ctypes.data_as(_c_dbl_p))
        self._check(rc, "dynconv")
        return y

    def select(self, logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids, k: int) -> SelectResult:
        """The whole selector. logits [B,L,V], hidden [B,L,H], W_sel [H,r], codebooks [V,r]."""
        logits = np.ascontiguousarray(logits)
        hidden = np.ascontiguousarray(hidden)
        W_sel = np.ascontiguousarray(W_sel)
        pred_cb = np.ascontiguousarray(pred_cb)
        succ_cb = np.ascontiguousarray(succ_cb)
        anchor_ids = np.ascontiguousarray(anchor_ids, dtype=np.int32)
        B, L, V = logits.shape
        H = hidden.shape[-1]
        r = W_sel.shape[1]
        if hidden.shape != (B, L, H) or W_sel.shape != (H, r) or pred_cb.shape != (V, r) \
                or succ_cb.shape != (V, r) or anchor_ids.shape != (B,):
            raise ValueError("inconsistent shapes")
        if hidden.dtype != W_sel.dtype or pred_cb.dtype != succ_cb.dtype:
            raise TypeError("hidden/W_sel and pred_cb/succ_cb share a dtype")
        out = SelectResult(np.zeros((B, L, k), np.int32), np.zeros((B, L, k)),
                           np.zeros((B, L, k, k)), np.zeros((B, L), np.int32), np.zeros((B, L)),
                           np.zeros((B, L), np.int32), np.zeros((B, L)), np.zeros((B,)))
        rc = self.lib.dflash2_ref_select(
            _ptr(logits), dtype_code(logits), _ptr(hidden), dtype_code(hidden), _ptr(W_sel),
            _ptr(pred_cb), _ptr(succ_cb), dtype_code(pred_cb), anchor_ids.ctypes.data_as(_c_int_p),
            B, L, V, H, r, k,
            out.cand_ids.ctypes.data_as(_c_int_p), out.unary.ctypes.data_as(_c_dbl_p),
            out.edges.ctypes.data_as(_c_dbl_p), out.path.ctypes.data_as(_c_int_p),
            out.lse.ctypes.data_as(_c_dbl_p), out.path_idx.ctypes.data_as(_c_int_p),
            out.margin.ctypes.data_as(_c_dbl_p), out.score.ctypes.data_as(_c_dbl_p))
        self._check(rc, "select")
        return out


_default: Oracle | None = None


def default() -> Oracle:
    """The oracle built from this directory's source (compiled on first use if absent)."""
    global _default
    if _default is None:
        _default = Oracle(LIBRARY)
    return _default
