"""The fused LM-head top-k pass (dflash2_lmhead_topk) vs the oracle (needs an MI355X).

Inputs come from synth.lmhead_inputs (bf16 hidden rows and an [V, H] bf16 LM-head weight). The
oracle computes the logits in fp64 from the same stored bits; the GPU accumulates the exact bf16
products in fp32 (v_mfma_f32_16x16x32_bf16: 32 products per MFMA, 2 ceil(H/64) MFMAs), so each of
its logits is within eps_v = (2 ceil(H/64) + 32) * 2^-24 * sum_h |hidden_h W_vh| of the exact one
(every fp32 rounding of a partial sum errs by at most 2^-24 times the sum of the magnitudes so
far, counted here against the whole sum). The checks, with the oracle's logits x and lse:
  * lse: |lse_gpu - lse| <= 1e-5 + 1e-4 |lse| + max_v eps_v;
  * ids: distinct and in range; every GPU id v has x_v >= x_(k) - 2 eps (x_(k): the oracle's k-th
    logit); every token with x_v > x_(k) + 2 eps is among the GPU ids; consecutive GPU ids are in
    candidate order up to 2 eps; where the oracle's logits are more than 2 eps apart around the
    k-th place the ids are exactly the oracle's, in order;
  * unary: |unary_gpu - (x_v - lse)| <= 1e-5 + 1e-4 |ref| + eps_v + max_v eps_v.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def lib():
    import dflash2_draft_candidate_amd as d2
    return d2


@pytest.fixture(scope="module")
def ref():
    return oracle.default()


def widen(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def check_rows(gpu, want, hidden, W, k, rows=None):
    ids_g, un_g, lse_g = gpu
    ids_r, un_r, lse_r, x = want
    rows = range(ids_r.shape[0]) if rows is None else rows
    H = hidden.shape[1]
    steps = 2 * -(-H // 64)
    ah = np.abs(widen(hidden))
    scale = np.empty((hidden.shape[0], W.shape[0]))   # sum_h |hidden_h W_vh|, in chunks of V
    for v0 in range(0, W.shape[0], 8192):
        scale[:, v0:v0 + 8192] = ah @ np.abs(widen(W[v0:v0 + 8192])).T
    eps = (steps + 32) * 2.0 ** -24 * scale
    V = W.shape[0]
    exact_rows = 0
    for i_ref, i in enumerate(rows):
        xi, ei = x[i_ref], eps[i_ref]
        emax = float(ei.max())
        assert abs(lse_g[i] - lse_r[i_ref]) <= 1e-5 + 1e-4 * abs(lse_r[i_ref]) + emax, \
            f"row {i}: lse {lse_g[i]} vs {lse_r[i_ref]}"
        g = ids_g[i].astype(np.int64)
        assert len(set(g.tolist())) == k and g.min() >= 0 and g.max() < V, f"row {i}: bad ids {g}"
        order = np.lexsort((np.arange(V), -xi))
        xk = xi[order[k - 1]]
        band = 2 * emax
        assert np.all(xi[g] >= xk - band), f"row {i}: an id below the k-th place"
        must = np.nonzero(xi > xk + band)[0]
        assert set(must.tolist()) <= set(g.tolist()), f"row {i}: a clear top-k token is missing"
        assert np.all(np.diff(xi[g]) <= band), f"row {i}: ids out of candidate order"
        gaps = np.abs(np.diff(xi[order[:k + 1]]))
        if gaps.min() > band:
            assert np.array_equal(g, order[:k]), f"row {i}: ids differ from the oracle's"
            exact_rows += 1
        want_u = xi[g] - lse_r[i_ref]
        tol = 1e-5 + 1e-4 * np.abs(want_u) + ei[g] + emax
        assert np.all(np.abs(un_g[i] - want_u) <= tol), f"row {i}: unary off by " \
            f"{np.max(np.abs(un_g[i] - want_u))}"
    return exact_rows


CASES = [
    # R, H, V, k, seed (R <= 16: one row tile; larger R is refused)
    (5, 64, 300, 4, 1),
    (13, 200, 1111, 16, 2),     # ragged rows, H not a multiple of 32, ragged V
    (16, 1024, 20011, 16, 3),
    (16, 128, 16, 16, 4),       # V = k: one 16-column tile, most waves without a tile
    (1, 8, 100, 1, 5),          # one row, one step, k = 1
    (16, 256, 3000, 8, 6),
    (9, 96, 4099, 16, 7),
    (16, 4104, 2500, 16, 8),    # 9 chunks of 512 h: wave 0 takes two, the others one
    (7, 8200, 1500, 8, 9),      # 17 chunks, the last of 8 h: two or three per wave
    (3, 64, 5, 5, 10),          # fewer vocabulary rows than one tile (k = V)
    (16, 520, 17, 16, 11),      # two tiles, the second of one row; H a 512-h chunk plus 8
]


@pytest.mark.parametrize("R,H,V,k,seed", CASES)
def test_lmhead_topk(lib, ref, R, H, V, k, seed):
    log(f"[lmhead] R={R} H={H} V={V} k={k}")
    hidden, W = synth.lmhead_inputs(R, H, V, 900 + seed)
    out = lib.lmhead_topk(synth.as_torch(hidden, DEV), synth.as_torch(W, DEV), k)
    torch.cuda.synchronize()
    gpu = tuple(synth.from_torch(t) for t in out)
    want = ref.lmhead_topk(hidden, W, k, want_logits=True)
    exact = check_rows(gpu, want, hidden, W, k)
    log(f"[lmhead] rows with exact ids: {exact}/{R}")


def test_lmhead_full_size(lib, ref):
    s = synth.LM_CONFIGS["lmhead-qwen3-8b-b1"]
    log(f"[lmhead] {s.name}: R={s.R} H={s.H} V={s.V} k={s.k} (every row against the oracle)")
    hidden, W = synth.lmhead_inputs(s.R, s.H, s.V, s.seed)
    out = lib.lmhead_topk(synth.as_torch(hidden, DEV), synth.as_torch(W, DEV), s.k)
    torch.cuda.synchronize()
    gpu = tuple(synth.from_torch(t) for t in out)
    want = ref.lmhead_topk(hidden, W, s.k, want_logits=True)
    exact = check_rows(gpu, want, hidden, W, s.k)
    log(f"[lmhead] rows with exact ids: {exact}/{s.R}")


def test_lmhead_refuses_more_rows(lib):
    hidden, W = synth.lmhead_inputs(17, 64, 300, 3)
    with pytest.raises(lib.Dflash2Error):
        lib.lmhead_topk(synth.as_torch(hidden, DEV), synth.as_torch(W, DEV), 4)


def test_lmhead_repeatable(lib):
    hidden, W = synth.lmhead_inputs(16, 512, 9000, 77)
    h, w = synth.as_torch(hidden, DEV), synth.as_torch(W, DEV)
    a = [synth.from_torch(t) for t in lib.lmhead_topk(h, w, 16)]
    b = [synth.from_torch(t) for t in lib.lmhead_topk(h, w, 16)]
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "the fused pass is deterministic"
