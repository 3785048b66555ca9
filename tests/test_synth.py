"""The seeded input generator (CPU only): determinism, the published generator definitions, and
the structure each workload promises."""
import math

import numpy as np
import torch

import synth

M64 = (1 << 64) - 1


def _mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _bits(seed, stream, i):
    key = _mix64((seed + 0x9E3779B97F4A7C15) & M64)
    key = _mix64(key ^ ((stream * 0xD1B54A32D192ED03) & M64))
    return _mix64((key + (i + 1) * 0x9E3779B97F4A7C15) & M64)


def test_splitmix64_reference_values():
    # the splitmix64 output function on state 0x9E3779B97F4A7C15 (first output of seed 0)
    assert _mix64(0x9E3779B97F4A7C15) == 0xE220A8397B1DCDAF
    for i in range(5):
        assert synth.lib().synth_bits(7, 3, i) == _bits(7, 3, i)


def test_normal_matches_box_muller_definition():
    seed, stream = 99, 4
    got = synth.normal(seed, stream, 10, std=2.0, mean=1.0)
    for i in range(10):
        u1 = ((_bits(seed, stream, 2 * (i // 2)) >> 11) + 0.5) / 2.0 ** 53
        u2 = ((_bits(seed, stream, 2 * (i // 2) + 1) >> 11) + 0.5) / 2.0 ** 53
        rad = math.sqrt(-2.0 * math.log(u1))
        z = rad * (math.sin if i % 2 else math.cos)(2 * math.pi * u2)
        assert got[i] == np.float32(1.0 + 2.0 * z)


def test_counter_based_offsets():
    full = synth.normal(5, 1, 1000)
    part = synth.normal(5, 1, 300, offset=500)
    assert np.array_equal(full[500:800], part)


def test_normal_moments():
    x = synth.normal(1, 1, 200000, std=3.0).astype(np.float64)
    assert abs(x.mean()) < 0.03 and abs(x.std() - 3.0) < 0.03


def test_bf16_rounding_matches_torch():
    x = synth.normal(2, 2, 100000, std=10.0)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]   # exact halfway cases
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16(x), want)


def test_distinct_ids():
    ids = synth.distinct_ids(3, 2, 50, 40, 36)
    assert ids.shape == (50, 36)
    for row in ids:
        assert len(set(row.tolist())) == 36 and row.min() >= 0 and row.max() < 40


def test_workloads_deterministic():
    a = synth.make_inputs("tiny")
    b = synth.make_inputs("tiny")
    for f in ("logits", "hidden", "W_sel", "pred_cb", "succ_cb", "anchor_ids"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


def test_workload_shapes_and_dtypes():
    s = synth.spec("serving-b64", B=2)
    x = synth.make_inputs(s)
    assert x.logits.shape == (2, 16, 151936) and x.logits.dtype == np.uint16
    assert x.hidden.shape == (2, 16, 4096) and x.W_sel.shape == (4096, 64)
    assert x.pred_cb.shape == (151936, 64) and x.anchor_ids.shape == (2,)
    # per-sequence seeds: sequence 0 of B=2 equals sequence 0 of B=1
    y = synth.make_inputs(synth.spec("serving-b64", B=1))
    assert np.array_equal(x.logits[0], y.logits[0]) and not np.array_equal(x.logits[0], x.logits[1])
    assert (x.anchor_ids >= 0).all() and (x.anchor_ids < 151936).all()


def _order(row: np.ndarray) -> np.ndarray:
    """Ids of the row in the candidate order: larger value first, lower id first on ties."""
    return np.lexsort((np.arange(row.size), -row.astype(np.float64)))


def test_stress_recipe():
    # near-flat and peaked rows as stated, with exact ties planted at ranks 0 (flat rows only),
    # floor(k/2) and k-1; the rank k-1 pair straddles the k-th place
    s = synth.spec("stress", B=2)
    x = synth.make_inputs(s)
    k = s.k
    for b in range(2):
        for p in range(s.L):
            row = x.logits[b, p].astype(np.float64)
            order = _order(row)
            flat = (b * s.L + p) % 2 == 0
            if flat:
                assert np.abs(row).max() < 1.0   # N(0, 0.1^2): no planted outliers
                assert row[order[0]] == row[order[1]]   # the copied maximum
            else:
                assert row[order[0]] > 11.0 and row[order[1]] < 1.0   # one token +12
            assert row[order[k // 2]] in (row[order[k // 2 - 1]], row[order[k // 2 + 1]])
            # the k-th and (k+1)-th place hold equal values: the tie straddles the boundary
            assert row[order[k - 1]] == row[order[k]], (b, p)
            assert order[k - 1] < order[k]


def test_stress_ties_straddle_both_ways():
    # across rows the planted copy at the k-th place lands on either side of the original
    # token's id: a copy with the lower id displaces the original from the top k, one with the
    # higher id stays just outside it. The copies are the tokens that differ from the unplanted
    # base row (same seeded streams, before any tie is planted).
    s = synth.spec("stress", B=8)
    x = synth.make_inputs(s)
    displaced = kept = 0
    for b in range(s.B):
        sb = synth.sequence_seed(s.seed, b)
        base = synth.normal(sb, synth.S_LOGITS, s.L * s.V, std=0.1).reshape(s.L, s.V)
        peak = synth.index(sb, synth.S_BOOST_IDS, s.L, s.V)
        for p in range(s.L):
            row = x.logits[b, p]
            if (b * s.L + p) % 2:
                base[p, peak[p]] += np.float32(12.0)
            copies = set(np.nonzero(row != base[p])[0].tolist())
            order = _order(row)
            pair = {int(order[s.k - 1]), int(order[s.k])}
            copy = pair & copies
            assert len(copy) == 1, (b, p)   # one of the straddling pair is a planted copy
            if copy == {int(order[s.k - 1])}:
                displaced += 1
            else:
                kept += 1
    assert displaced > 0 and kept > 0


def test_ladder_planted_ties():
    s = synth.spec("stress", B=2, recipe="ladder")
    x = synth.make_inputs(s)
    k = s.k
    for b in range(2):
        for p in range(s.L):
            row = x.logits[b, p]
            if (b * s.L + p) % 2 == 0:
                # 8 tokens at exactly 1.0 and a tied pair at the top of the ladder
                assert (row == 1.0).sum() == 8
                top = row.max()
                assert (row == top).sum() == 2 and top == 1.0 + 0.125 * (k - 4)
            else:
                top = row.max()
                assert (row == top).sum() == 2 and top > 11.0


def test_gemma_zipf_boosts():
    s = synth.spec("gemma4-31b", B=1, L=2)
    x = synth.make_inputs(s)
    v = synth.bf16_to_f32(x.logits[0, 0]).astype(np.float64)
    assert v.max() > 6.0   # the rank-1 boost (8) sits on top of N(0, 2^2) noise
