"""MI355X (gfx950) DFlash 2 candidate selector: Python binding over the C ABI of libdflash2.so.

This module only marshals arguments: it checks shapes and dtypes, allocates outputs and
workspace with torch on the inputs' device, and passes raw pointers plus the current HIP stream
to the library. Every step of the selector runs in the library's HIP kernels. If the built
library is missing, importing this package raises ImportError; there is no fallback.

    cand_ids, unary, edges, path = select(logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids, k)

Shapes: logits [B, L, V] (float32 or bfloat16), hidden [B, L, H] and W_sel [H, r] (one dtype),
pred_cb / succ_cb [V, r] (one dtype), anchor_ids [B] int32. See include/dflash2.h.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime first, so libdflash2 binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "libdflash2.so")

if not os.path.exists(LIBRARY):
    raise ImportError(f"{LIBRARY} is not built; run `python -c 'import __graft_entry__ as g; "
                      "g.build()'` or `python dflash2_draft_candidate_amd/build.py`")
_lib = ctypes.CDLL(LIBRARY)

F32, BF16 = 0, 1
OK = 0
MAX_K = 64
MAX_R = 256
LMHEAD_MAX_K = 16

_vp, _ci, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_lib.dflash2_version.restype = _ci
_lib.dflash2_status_string.argtypes = [_ci]
_lib.dflash2_status_string.restype = ctypes.c_char_p
_lib.dflash2_workspace_bytes.argtypes = [_ci] * 6
_lib.dflash2_workspace_bytes.restype = _sz
_lib.dflash2_select.argtypes = [_vp, _ci, _vp, _ci, _vp, _vp, _vp, _ci, _vp] + [_ci] * 6 + \
    [_vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dflash2_select.restype = _ci
_lib.dflash2_select_noalloc.argtypes = [_vp, _ci, _vp, _ci, _vp, _vp, _vp, _ci, _vp] + \
    [_ci] * 6 + [_vp, _vp, _vp, _vp, _vp]
_lib.dflash2_select_noalloc.restype = _ci
_lib.dflash2_topk_lse_workspace_bytes.argtypes = [_ci] * 4
_lib.dflash2_topk_lse_workspace_bytes.restype = _sz
_lib.dflash2_topk_lse.argtypes = [_vp, _ci, _ci, _ci, _ci, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dflash2_topk_lse.restype = _ci
_lib.dflash2_gate_workspace_bytes.argtypes = [_ci] * 3
_lib.dflash2_gate_workspace_bytes.restype = _sz
_lib.dflash2_gate.argtypes = [_vp, _vp, _ci, _ci, _ci, _ci, _vp, _vp, _sz, _vp]
_lib.dflash2_gate.restype = _ci
_lib.dflash2_lattice.argtypes = [_vp, _vp, _vp, _vp, _vp, _ci, _vp] + [_ci] * 5 + [_vp, _vp]
_lib.dflash2_lattice.restype = _ci
_lib.dflash2_walk.argtypes = [_vp, _vp, _ci, _ci, _ci, _vp, _vp, _vp]
_lib.dflash2_walk.restype = _ci
_cf = ctypes.c_float
_lib.dflash2_walk_ex.argtypes = [_vp, _vp, _ci, _ci, _ci, _cf, _vp, _cf, _vp, _vp, _vp, _vp]
_lib.dflash2_walk_ex.restype = _ci
_lib.dflash2_select_ex.argtypes = [_vp, _ci, _vp, _ci, _vp, _vp, _vp, _ci, _vp] + [_ci] * 6 + \
    [_cf, _vp, _cf, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.dflash2_select_ex.restype = _ci
_lib.dflash2_dynconv.argtypes = [_vp, _vp, _vp, _ci, _ci, _ci, _ci, _ci, _ci, _vp, _vp]
_lib.dflash2_dynconv.restype = _ci
_lib.dflash2_lmhead_topk_workspace_bytes.argtypes = [_ci] * 4
_lib.dflash2_lmhead_topk_workspace_bytes.restype = _sz
_lib.dflash2_lmhead_topk.argtypes = [_vp, _vp] + [_ci] * 4 + [_vp, _vp, _vp, _vp, _sz, _vp]
_lib.dflash2_lmhead_topk.restype = _ci

EXPORTS = ("dflash2_version", "dflash2_status_string", "dflash2_workspace_bytes",
           "dflash2_select", "dflash2_select_noalloc", "dflash2_topk_lse_workspace_bytes", "dflash2_topk_lse",
           "dflash2_gate_workspace_bytes", "dflash2_gate", "dflash2_lattice", "dflash2_walk",
           "dflash2_select_ex", "dflash2_walk_ex", "dflash2_dynconv",
           "dflash2_lmhead_topk_workspace_bytes", "dflash2_lmhead_topk")


class Dflash2Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_lib.dflash2_status_string(status).decode()} (status {status})")
        self.status = status


def library():
    """The loaded ctypes library (for tests that call the C ABI directly)."""
    return _lib


def version() -> int:
    return _lib.dflash2_version()


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


# Every entry point declares its pointer arguments as c_void_p, so plain integers (and None for
# NULL) are passed as they are: no ctypes object is built per argument.
def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device) -> int:
    """The current stream of `device` as a raw handle."""
    index = device.index if device.index is not None else torch.cuda.current_device()
    if _raw_stream is not None:
        return _raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream


def _check(rc: int, what: str):
    if rc != OK:
        raise Dflash2Error(rc, what)


def _contig(*ts: torch.Tensor):
    for t in ts:
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def workspace_bytes(B: int, L: int, V: int, H: int, r: int, k: int) -> int:
    return int(_lib.dflash2_workspace_bytes(B, L, V, H, r, k))


def select(logits: torch.Tensor, hidden: torch.Tensor, W_sel: torch.Tensor,
           pred_cb: torch.Tensor, succ_cb: torch.Tensor, anchor_ids: torch.Tensor, k: int,
           out: tuple | None = None, workspace: torch.Tensor | None = None):
    """The whole selector. Returns (cand_ids [B,L,k] int32, unary [B,L,k] f32,
    edges [B,L,k,k] f32, path [B,L] int32). `out` / `workspace` may be passed to reuse buffers."""
    _contig(logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids)
    B, L, V = logits.shape
    H = hidden.shape[-1]
    r = W_sel.shape[1]
    if hidden.shape != (B, L, H) or W_sel.shape != (H, r) or pred_cb.shape != (V, r) \
            or succ_cb.shape != (V, r) or anchor_ids.shape != (B,):
        raise ValueError("inconsistent shapes")
    if hidden.dtype != W_sel.dtype or pred_cb.dtype != succ_cb.dtype:
        raise TypeError("hidden/W_sel and pred_cb/succ_cb must share a dtype")
    if anchor_ids.dtype != torch.int32:
        raise TypeError("anchor_ids must be int32")
    dev = logits.device
    if out is None:
        out = (torch.empty((B, L, k), dtype=torch.int32, device=dev),
               torch.empty((B, L, k), dtype=torch.float32, device=dev),
               torch.empty((B, L, k, k), dtype=torch.float32, device=dev),
               torch.empty((B, L), dtype=torch.int32, device=dev))
    cand_ids, unary, edges, path = out
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, L, V, H, r, k), dev)
    rc = _lib.dflash2_select(_ptr(logits), _dtype(logits), _ptr(hidden), _dtype(hidden),
                             _ptr(W_sel), _ptr(pred_cb), _ptr(succ_cb), _dtype(pred_cb),
                             _ptr(anchor_ids), B, L, V, H, r, k, _ptr(cand_ids), _ptr(unary),
                             _ptr(edges), _ptr(path), _ptr(workspace), workspace.numel(),
                             _stream(dev))
    _check(rc, "dflash2_select")
    return cand_ids, unary, edges, path


NOALLOC_SCRATCH_BYTES = 16 << 20


def select_noalloc(logits: torch.Tensor, hidden: torch.Tensor, W_sel: torch.Tensor,
                   pred_cb: torch.Tensor, succ_cb: torch.Tensor, anchor_ids: torch.Tensor, k: int,
                   out: tuple):
    """dflash2_select_noalloc: the whole selector on the library's per-GPU scratch array instead
    of a workspace. `out` = (cand_ids, unary, edges, path), preallocated as for select()."""
    _contig(logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids)
    B, L, V = logits.shape
    H = hidden.shape[-1]
    r = W_sel.shape[1]
    if hidden.shape != (B, L, H) or W_sel.shape != (H, r) or pred_cb.shape != (V, r) \
            or succ_cb.shape != (V, r) or anchor_ids.shape != (B,):
        raise ValueError("inconsistent shapes")
    if hidden.dtype != W_sel.dtype or pred_cb.dtype != succ_cb.dtype:
        raise TypeError("hidden/W_sel and pred_cb/succ_cb must share a dtype")
    if anchor_ids.dtype != torch.int32:
        raise TypeError("anchor_ids must be int32")
    cand_ids, unary, edges, path = out
    rc = _lib.dflash2_select_noalloc(_ptr(logits), _dtype(logits), _ptr(hidden), _dtype(hidden),
                                     _ptr(W_sel), _ptr(pred_cb), _ptr(succ_cb), _dtype(pred_cb),
                                     _ptr(anchor_ids), B, L, V, H, r, k, _ptr(cand_ids),
                                     _ptr(unary), _ptr(edges), _ptr(path), _stream(logits.device))
    _check(rc, "dflash2_select_noalloc")
    return cand_ids, unary, edges, path


def select_ex(logits: torch.Tensor, hidden: torch.Tensor, W_sel: torch.Tensor,
              pred_cb: torch.Tensor, succ_cb: torch.Tensor, anchor_ids: torch.Tensor, k: int,
              temperature: float = 0.0, uniforms: torch.Tensor | None = None, p_min: float = 0.0,
              out: tuple | None = None, workspace: torch.Tensor | None = None):
    """The selector with the walk's sampling (temperature > 0, uniforms [B,L] float32 in [0,1))
    and p_min early stop. Returns (cand_ids, unary, edges, path, draft_len [B] int32)."""
    _contig(logits, hidden, W_sel, pred_cb, succ_cb, anchor_ids)
    B, L, V = logits.shape
    H = hidden.shape[-1]
    r = W_sel.shape[1]
    if hidden.shape != (B, L, H) or W_sel.shape != (H, r) or pred_cb.shape != (V, r) \
            or succ_cb.shape != (V, r) or anchor_ids.shape != (B,):
        raise ValueError("inconsistent shapes")
    if hidden.dtype != W_sel.dtype or pred_cb.dtype != succ_cb.dtype:
        raise TypeError("hidden/W_sel and pred_cb/succ_cb must share a dtype")
    if anchor_ids.dtype != torch.int32:
        raise TypeError("anchor_ids must be int32")
    if uniforms is not None:
        _contig(uniforms)
        if uniforms.shape != (B, L) or uniforms.dtype != torch.float32:
            raise ValueError("uniforms must be [B, L] float32")
    dev = logits.device
    if out is None:
        out = (torch.empty((B, L, k), dtype=torch.int32, device=dev),
               torch.empty((B, L, k), dtype=torch.float32, device=dev),
               torch.empty((B, L, k, k), dtype=torch.float32, device=dev),
               torch.empty((B, L), dtype=torch.int32, device=dev),
               torch.empty((B,), dtype=torch.int32, device=dev))
    cand_ids, unary, edges, path, draft_len = out
    if workspace is None:
        workspace = _workspace(workspace_bytes(B, L, V, H, r, k), dev)
    rc = _lib.dflash2_select_ex(_ptr(logits), _dtype(logits), _ptr(hidden), _dtype(hidden),
                                _ptr(W_sel), _ptr(pred_cb), _ptr(succ_cb), _dtype(pred_cb),
                                _ptr(anchor_ids), B, L, V, H, r, k, float(temperature),
                                _ptr(uniforms), float(p_min), _ptr(cand_ids), _ptr(unary),
                                _ptr(edges), _ptr(path), _ptr(draft_len), _ptr(workspace),
                                workspace.numel(), _stream(dev))
    _check(rc, "dflash2_select_ex")
    return cand_ids, unary, edges, path, draft_len


def topk_lse(logits: torch.Tensor, k: int):
    """logits [R, V] -> (cand_ids [R,k] int32, unary [R,k] f32, lse [R] f32)."""
    _contig(logits)
    R, V = logits.shape
    dev = logits.device
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    unary = torch.empty((R, k), dtype=torch.float32, device=dev)
    lse = torch.empty((R,), dtype=torch.float32, device=dev)
    ws = _workspace(_lib.dflash2_topk_lse_workspace_bytes(R, V, k, _dtype(logits)), dev)
    rc = _lib.dflash2_topk_lse(_ptr(logits), _dtype(logits), R, V, k, _ptr(ids), _ptr(unary),
                               _ptr(lse), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "dflash2_topk_lse")
    return ids, unary, lse


LMHEAD_MAX_ROWS = 16  # DFLASH2_LMHEAD_MAX_ROWS


def lmhead_topk(hidden: torch.Tensor, W_lm: torch.Tensor, k: int):
    """hidden [R, H] bf16, W_lm [V, H] bf16 -> (cand_ids [R,k] int32, unary [R,k] f32, lse [R]
    f32) of the top-k pass over hidden . W_lm^T, computed without materialising the logits."""
    _contig(hidden, W_lm)
    R, H = hidden.shape
    V = W_lm.shape[0]
    if W_lm.shape[1] != H or hidden.dtype != torch.bfloat16 or W_lm.dtype != torch.bfloat16:
        raise ValueError("hidden [R, H] and W_lm [V, H], both bfloat16")
    dev = hidden.device
    ids = torch.empty((R, k), dtype=torch.int32, device=dev)
    unary = torch.empty((R, k), dtype=torch.float32, device=dev)
    lse = torch.empty((R,), dtype=torch.float32, device=dev)
    if R > LMHEAD_MAX_ROWS:
        raise Dflash2Error(-2, f"dflash2_lmhead_topk: R = {R} rows (at most {LMHEAD_MAX_ROWS}: "
                               "use a product and topk_lse)")
    need = _lib.dflash2_lmhead_topk_workspace_bytes(R, H, V, k)
    if need == 0:
        raise Dflash2Error(-1, "dflash2_lmhead_topk: invalid sizes")
    ws = _workspace(need, dev)
    rc = _lib.dflash2_lmhead_topk(_ptr(hidden), _ptr(W_lm), R, H, V, k, _ptr(ids), _ptr(unary),
                                  _ptr(lse), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "dflash2_lmhead_topk")
    return ids, unary, lse


def gate(hidden: torch.Tensor, W_sel: torch.Tensor):
    """hidden [R, H], W_sel [H, r] -> g [R, r] f32."""
    _contig(hidden, W_sel)
    R, H = hidden.shape
    r = W_sel.shape[1]
    if W_sel.shape[0] != H or hidden.dtype != W_sel.dtype:
        raise ValueError("W_sel must be [H, r] with hidden's dtype")
    dev = hidden.device
    g = torch.empty((R, r), dtype=torch.float32, device=dev)
    ws = _workspace(_lib.dflash2_gate_workspace_bytes(R, H, r), dev)
    rc = _lib.dflash2_gate(_ptr(hidden), _ptr(W_sel), _dtype(hidden), R, H, r, _ptr(g), _ptr(ws),
                           ws.numel(), _stream(dev))
    _check(rc, "dflash2_gate")
    return g


def lattice(cand_ids: torch.Tensor, unary: torch.Tensor, g: torch.Tensor, pred_cb: torch.Tensor,
            succ_cb: torch.Tensor, anchor_ids: torch.Tensor):
    """cand_ids/unary [B,L,k], g [B,L,r] f32, codebooks [V,r], anchor_ids [B] -> edges."""
    _contig(cand_ids, unary, g, pred_cb, succ_cb, anchor_ids)
    B, L, k = cand_ids.shape
    V, r = pred_cb.shape
    if cand_ids.dtype != torch.int32 or anchor_ids.dtype != torch.int32 or \
            unary.dtype != torch.float32 or g.dtype != torch.float32:
        raise TypeError("cand_ids/anchor_ids int32, unary/g float32")
    if g.shape != (B, L, r) or unary.shape != (B, L, k) or succ_cb.shape != (V, r) or \
            succ_cb.dtype != pred_cb.dtype:
        raise ValueError("inconsistent shapes")
    dev = cand_ids.device
    edges = torch.empty((B, L, k, k), dtype=torch.float32, device=dev)
    rc = _lib.dflash2_lattice(_ptr(cand_ids), _ptr(unary), _ptr(g), _ptr(pred_cb), _ptr(succ_cb),
                              _dtype(pred_cb), _ptr(anchor_ids), B, L, V, r, k, _ptr(edges),
                              _stream(dev))
    _check(rc, "dflash2_lattice")
    return edges


def walk(edges: torch.Tensor, cand_ids: torch.Tensor):
    """edges [B,L,k,k] f32, cand_ids [B,L,k] int32 -> (path [B,L] int32, path_idx [B,L] int32)."""
    _contig(edges, cand_ids)
    B, L, k = cand_ids.shape
    if edges.shape != (B, L, k, k) or edges.dtype != torch.float32 or cand_ids.dtype != torch.int32:
        raise ValueError("edges [B,L,k,k] float32, cand_ids [B,L,k] int32")
    dev = edges.device
    path = torch.empty((B, L), dtype=torch.int32, device=dev)
    idx = torch.empty((B, L), dtype=torch.int32, device=dev)
    rc = _lib.dflash2_walk(_ptr(edges), _ptr(cand_ids), B, L, k, _ptr(path), _ptr(idx),
                           _stream(dev))
    _check(rc, "dflash2_walk")
    return path, idx


def walk_ex(edges: torch.Tensor, cand_ids: torch.Tensor, temperature: float = 0.0,
            uniforms: torch.Tensor | None = None, p_min: float = 0.0):
    """The walk with sampling and the p_min stop -> (path [B,L], path_idx [B,L], draft_len [B])."""
    _contig(edges, cand_ids)
    B, L, k = cand_ids.shape
    if edges.shape != (B, L, k, k) or edges.dtype != torch.float32 or cand_ids.dtype != torch.int32:
        raise ValueError("edges [B,L,k,k] float32, cand_ids [B,L,k] int32")
    if uniforms is not None:
        _contig(uniforms)
        if uniforms.shape != (B, L) or uniforms.dtype != torch.float32:
            raise ValueError("uniforms must be [B, L] float32")
    dev = edges.device
    path = torch.empty((B, L), dtype=torch.int32, device=dev)
    idx = torch.empty((B, L), dtype=torch.int32, device=dev)
    dlen = torch.empty((B,), dtype=torch.int32, device=dev)
    rc = _lib.dflash2_walk_ex(_ptr(edges), _ptr(cand_ids), B, L, k, float(temperature),
                              _ptr(uniforms), float(p_min), _ptr(path), _ptr(idx), _ptr(dlen),
                              _stream(dev))
    _check(rc, "dflash2_walk_ex")
    return path, idx, dlen


def dynconv(x: torch.Tensor, base: torch.Tensor, dyn: torch.Tensor, group: int,
            out: torch.Tensor | None = None):
    """Grouped dynamic depthwise convolution of the draft blocks: x [nb,T,C], base [K,C],
    dyn [nb,T,K,C/group] (one dtype) -> y [nb,T,C] of x's dtype."""
    _contig(x, base, dyn)
    nb, T, C = x.shape
    K = base.shape[0]
    if base.shape != (K, C) or C % group != 0 or dyn.shape != (nb, T, K, C // group):
        raise ValueError("inconsistent shapes")
    if base.dtype != x.dtype or dyn.dtype != x.dtype:
        raise TypeError("x, base and dyn must share a dtype")
    y = torch.empty_like(x) if out is None else out
    rc = _lib.dflash2_dynconv(_ptr(x), _ptr(base), _ptr(dyn), _dtype(x), nb, T, C, K, group,
                              _ptr(y), _stream(x.device))
    _check(rc, "dflash2_dynconv")
    return y
