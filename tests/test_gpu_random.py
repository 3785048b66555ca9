"""Seeded random shapes through the selector and its stages vs the oracle (needs an MI355X).

The fixed parity cases pick shapes by hand; this sweep draws 32 small ones from a fixed seed, mixing
every size the kernels treat differently: one or many sequences, block lengths across the walk's
passes, vocabularies from a few tokens to several chunks per wave, k from 1 to 64, ranks from 1 to
256 (ragged rank chunks, one to four gate column tiles), fp32 and bf16 storage of each input, and
every logit recipe of the input generator. Checks are the same as for the fixed cases: cand_ids
bit-exact, unary and edges within 1e-5 abs + 1e-4 rel, the path identical wherever the oracle's
best successor wins by more than 1e-3. The stand-alone entry points (top-k pass, gate, lattice,
walk modes, convolution, LM-head pass) get random shapes of their own, checked by the same code
as their fixed cases.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import test_gpu_lmhead as LM
import test_gpu_parity as P
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


def _stage_cases(seed: int) -> dict:
    rng = np.random.default_rng(seed)
    pick = lambda a: a[int(rng.integers(0, len(a)))]
    logit_cases = ["normal", "ties", "signed_zero", "constant", "ascending", "descending",
                   "peaked", "high", "low", "mixed_range", "wide"]
    c = {"topk": [], "gate": [], "lattice": [], "walk_ex": [], "conv": [], "lm": []}
    for _ in range(12):
        V = int(pick([1, 2, 5, 63, 64, 65, 1000, 4097, 20011, 70001, 151936, 262144]))
        R = int(pick([1, 2, 3, 7, 16, 64, 129, 600, 1030]))
        while R * V > 4_000_000 and R > 1:
            R //= 2
        c["topk"].append((pick(logit_cases), R, V, int(min(V, pick([1, 2, 8, 16, 17, 32, 64]))),
                          pick(["f32", "bf16"])))
    for _ in range(6):
        c["gate"].append((int(pick([1, 3, 16, 65, 1024])), int(pick([8, 40, 100, 1024, 4096])),
                          int(pick([1, 16, 33, 64, 130, 256])), pick(["f32", "bf16"])))
        V = int(pick([10, 100, 1000, 151936]))
        c["lattice"].append((int(rng.integers(1, 9)), int(pick([1, 2, 5, 16, 33])), V,
                             int(pick([1, 5, 16, 64, 100, 256])),
                             int(min(V, pick([1, 3, 16, 17, 32, 64]))), pick(["f32", "bf16"])))
        G = int(pick([1, 2, 4, 5, 8, 16]))
        c["conv"].append((int(rng.integers(1, 65)), int(rng.integers(1, 34)),
                          G * int(pick([1, 2, 3, 8, 64, 256])), int(pick([1, 2, 3, 4, 8])), G,
                          pick(["f32", "bf16"])))
        V = int(pick([16, 17, 100, 1000, 4099, 20011]))
        c["lm"].append((int(pick([1, 5, 16, 3, 9, 13, 11])), int(pick([8, 64, 96, 200, 1024])),
                        V, int(min(V, pick([1, 4, 8, 15, 16]))), int(rng.integers(0, 1000))))
    for _ in range(8):
        c["walk_ex"].append((int(rng.integers(1, 9)), int(rng.integers(1, 41)),
                             int(pick([1, 2, 3, 16, 17, 33, 64])), float(pick([0.0, 0.3, 1.0, 2.0])),
                             float(pick([0.0, 0.05, 0.3, 0.9]))))
    return c


STAGES = _stage_cases(1202)
_ids = lambda cases: ["-".join(str(v) for v in c) for c in cases]


@pytest.mark.parametrize("args", STAGES["topk"], ids=_ids(STAGES["topk"]))
def test_topk_lse_random_shape(lib, ref, args):
    P.test_topk_lse(lib, ref, *args)


@pytest.mark.parametrize("args", STAGES["gate"], ids=_ids(STAGES["gate"]))
def test_gate_random_shape(lib, ref, args):
    P.test_gate(lib, ref, *args)


@pytest.mark.parametrize("args", STAGES["lattice"], ids=_ids(STAGES["lattice"]))
def test_lattice_random_shape(lib, ref, args):
    P.test_lattice(lib, ref, *args)


@pytest.mark.parametrize("args", STAGES["walk_ex"], ids=_ids(STAGES["walk_ex"]))
def test_walk_modes_random_shape(lib, ref, args):
    P.test_walk_ex(lib, ref, *args)


@pytest.mark.parametrize("args", STAGES["conv"], ids=_ids(STAGES["conv"]))
def test_dynconv_random_shape(lib, ref, args):
    P.test_dynconv(lib, ref, *args)


@pytest.mark.parametrize("args", STAGES["lm"], ids=_ids(STAGES["lm"]))
def test_lmhead_random_shape(lib, ref, args):
    LM.test_lmhead_topk(lib, ref, *args)
