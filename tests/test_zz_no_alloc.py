"""dflash2_select_noalloc (the library's per-GPU scratch array instead of a caller workspace) vs
dflash2_select on the same inputs (needs an MI355X). Both run the same kernels, so every output
must match bit for bit. Two calls in a row: the second on a smaller workload, after the first
left its contents in the shared array."""
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _args(x):
    t = lambda a: synth.as_torch(a, DEV)
    return (t(x.logits), t(x.hidden), t(x.W_sel), t(x.pred_cb), t(x.succ_cb), t(x.anchor_ids),
            x.spec.k)


def _out(s):
    return (torch.full((s.B, s.L, s.k), -7, dtype=torch.int32, device=DEV),
            torch.full((s.B, s.L, s.k), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((s.B, s.L, s.k, s.k), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((s.B, s.L), -7, dtype=torch.int32, device=DEV))


def test_select_noalloc_matches_select():
    import dflash2_draft_candidate_amd as d2
    # serving-b64, then qwen3-8b-b1 (fewer rows, sliced rows: slice partials in the array) and a
    # small fp32 case, each after the previous call's contents
    cases = [synth.spec("serving-b64"), synth.spec("qwen3-8b-b1"),
             synth.Spec("case", 3, 5, 7, 1021, 100, 24, "f32", "f32", "f32", "normal", 41)]
    for s in cases:
        log(f"select_noalloc {s.name}: B={s.B} L={s.L} V={s.V} k={s.k}")
        x = synth.make_inputs(s)
        args = _args(x)
        want = d2.select(*args)
        got = d2.select_noalloc(*args, out=_out(s))
        torch.cuda.synchronize()
        for a, b, what in zip(got, want, ("cand_ids", "unary", "edges", "path")):
            a, b = synth.from_torch(a), synth.from_torch(b)
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{s.name}: {what} differs"
