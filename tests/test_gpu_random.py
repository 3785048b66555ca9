"""Seeded random shapes through the whole selector (dflash2_select) vs the oracle (needs an MI355X).

The fixed parity cases pick shapes by hand; this sweep draws 32 small ones from a fixed seed, mixing
every size the kernels treat differently: one or many sequences, block lengths across the walk's
passes, vocabularies from a few tokens to several chunks per wave, k from 1 to 64, ranks from 1 to
256 (ragged rank chunks, one to four gate column tiles), fp32 and bf16 storage of each input, and
every logit recipe of the input generator. Checks are the same as for the fixed cases: cand_ids
bit-exact, unary and edges within 1e-5 abs + 1e-4 rel, the path identical wherever the oracle's
best successor wins by more than 1e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_select

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _random_specs(n: int, seed: int) -> list:
    rng = np.random.default_rng(seed)
    pick = lambda a: a[int(rng.integers(0, len(a)))]
    specs = []
    for i in range(n):
        B = int(rng.integers(1, 9))
        L = int(pick([1, 2, 3, 5, 8, 16, 17, 33]))
        recipe = pick(["normal", "stress", "zipf32", "boost8"])
        # the other recipes place up to max(k + 4, 34) distinct ids per row
        V = int(pick([7, 64, 257, 1000, 4099, 20011, 65536] if recipe == "normal"
                     else [257, 1000, 4099, 20011, 65536]))
        V = min(V, 2_000_000 // (B * L))
        k = int(min(V, pick([1, 3, 8, 16, 17, 32, 64])))
        H = int(pick([8, 40, 64, 200, 1024]))
        r = int(pick([1, 5, 16, 33, 64, 100, 128, 200, 256]))
        ld, ad, cd = (pick(["f32", "bf16"]) for _ in range(3))
        specs.append(synth.Spec(f"random{i}", B, L, k, V, H, r, ld, ad, cd, recipe, 5000 + i))
    return specs


RANDOM_SPECS = _random_specs(32, 20261202)


@pytest.fixture(scope="module")
def lib():
    import dflash2_draft_candidate_amd as d2
    return d2


@pytest.fixture(scope="module")
def ref():
    return oracle.default()


@pytest.mark.parametrize("s", RANDOM_SPECS,
                         ids=[f"{s.name}-B{s.B}-L{s.L}-V{s.V}-H{s.H}-r{s.r}-k{s.k}-"
                              f"{s.logits_dtype}{s.act_dtype}{s.cb_dtype}-{s.recipe}"
                              for s in RANDOM_SPECS])
def test_select_random_shape(lib, ref, s):
    print(f"select {s}", file=sys.stderr, flush=True)
    x = synth.make_inputs(s)
    T = lambda a: synth.as_torch(a, DEV)
    out = lib.select(T(x.logits), T(x.hidden), T(x.W_sel), T(x.pred_cb), T(x.succ_cb),
                     T(x.anchor_ids), s.k)
    torch.cuda.synchronize()
    gpu = tuple(synth.from_torch(t) for t in out)
    want = ref.select(x.logits, x.hidden, x.W_sel, x.pred_cb, x.succ_cb, x.anchor_ids, s.k)
    check_select(gpu, want)
