"""The selector captured in a HIP graph and replayed (needs an MI355X).

A captured launch keeps the launch epoch of its capture, and the top-k pass for few rows counts
slice arrivals in workspace counters that carry that epoch; the last slice of a row clears its
count, so a replay starts from zero. Each case captures dflash2_select on one input, replays it
several times with eager selector calls on the same workspace in between (their newer epochs
leave the counters to be re-based by the replay), and checks every replay against the eager
result on the same input bit for bit: the replay runs the same kernels.
"""
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


def _same(got, want, what):
    for a, b, name in zip(got, want, ("cand_ids", "unary", "edges", "path")):
        a, b = synth.from_torch(a), synth.from_torch(b)
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"{what}: {name} differs"


CASES = [
    # rows few enough for the one-round pass, sliced (in-kernel slice merge) with the gate fused
    synth.spec("qwen3-8b-b1"),
    # one slice per row (fp32)
    synth.spec("tiny"),
    # the streaming pass (256 rows)
    synth.Spec("rows256", 16, 16, 16, 4099, 64, 16, "bf16", "bf16", "bf16", "boost8", 77),
]


@pytest.mark.parametrize("s", CASES, ids=lambda s: s.name)
def test_select_graph_replay(s):
    import dflash2_draft_candidate_amd as d2
    log(f"graph {s.name}: B={s.B} L={s.L} V={s.V} k={s.k} {s.logits_dtype}")
    x = synth.make_inputs(s)
    other = synth.make_inputs(s, seed=s.seed + 1000)
    args, args_other = _args(x), _args(other)
    ws = torch.empty(max(16, d2.workspace_bytes(s.B, s.L, s.V, s.H, s.r, s.k)), dtype=torch.uint8,
                     device=DEV)
    want = [t.clone() for t in d2.select(*args, out=_out(s), workspace=ws)]
    want_other = [t.clone() for t in d2.select(*args_other, out=_out(s), workspace=ws)]
    torch.cuda.synchronize()
    out = _out(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d2.select(*args, out=out, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        for t, fill in zip(out, (-7, float("nan"), float("nan"), -7)):
            t.fill_(fill)
        g.replay()
        torch.cuda.synchronize()
        _same(out, want, f"{s.name} replay {rep}")
        # an eager call on the same workspace between replays (a newer launch epoch)
        _same(d2.select(*args_other, out=_out(s), workspace=ws), want_other,
              f"{s.name} eager after replay {rep}")
        torch.cuda.synchronize()
