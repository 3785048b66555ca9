"""Comparison rules between the HIP path and the oracle.

* cand_ids: bit-exact.
* unary, edges (and the gate g): |gpu - ref| <= ATOL + RTOL * |ref| with ref in fp64.
* path: walk the GPU's own path. At each position, in the oracle's lattice row of the GPU's
  previous choice, let margin = best - second best. Where margin > PATH_MARGIN the GPU must pick
  the oracle's argmax; where it is smaller the GPU's pick must lie within PATH_MARGIN of the best
  (a legal near-tie). When every margin exceeds PATH_MARGIN this is "paths identical".
"""
from __future__ import annotations

import numpy as np

ATOL = 1e-5
RTOL = 1e-4
PATH_MARGIN = 1e-3


def assert_close(gpu, ref, what: str, atol: float = ATOL, rtol: float = RTOL):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    err = np.abs(gpu - ref)
    tol = atol + rtol * np.abs(ref)
    bad = ~(err <= tol)  # NaN counts as bad
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {idx}:"
                             f" gpu={gpu[idx]!r} ref={ref[idx]!r} err={err[idx]:.3e}")


def assert_ids_equal(gpu, ref, what: str):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    if not np.array_equal(gpu, ref):
        bad = np.argwhere(gpu != ref)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches; first at {i}: gpu={gpu[i]} ref={ref[i]}")


def path_indices(path, cand_ids):
    """Candidate index j of each path token (ids within a row are distinct)."""
    B, L, k = cand_ids.shape
    idx = np.full((B, L), -1, np.int64)
    for b in range(B):
        for p in range(L):
            hit = np.nonzero(cand_ids[b, p] == path[b, p])[0]
            assert hit.size == 1, f"path token {path[b, p]} not among the candidates of ({b},{p})"
            idx[b, p] = hit[0]
    return idx


def check_path(gpu_path, cand_ids, ref_edges) -> int:
    """Margin-aware path rule; returns the number of near-tie steps that were exempt."""
    idx = path_indices(np.asarray(gpu_path), np.asarray(cand_ids))
    B, L = idx.shape
    exempt = 0
    for b in range(B):
        prev = 0
        for p in range(L):
            row = ref_edges[b, p, prev]
            best = int(np.argmax(row))   # lowest index on ties
            srt = np.sort(row)
            margin = np.inf if row.size == 1 else srt[-1] - srt[-2]
            j = idx[b, p]
            if margin > PATH_MARGIN:
                assert j == best, f"path ({b},{p}): gpu picked {j}, oracle {best}, margin {margin:.3e}"
            else:
                exempt += 1
                assert row[best] - row[j] <= PATH_MARGIN, f"path ({b},{p}): pick {j} not a near-tie"
            prev = j
    return exempt


def check_select(gpu, ref) -> int:
    """gpu = (cand_ids, unary, edges, path) as numpy; ref = oracle SelectResult."""
    cand, unary, edges, path = gpu
    assert_ids_equal(cand, ref.cand_ids, "cand_ids")
    assert_close(unary, ref.unary, "unary")
    assert_close(edges, ref.edges, "edges")
    return check_path(path, cand, ref.edges)
