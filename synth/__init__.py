"""Seeded synthetic workloads for the DFlash 2 candidate selector.

Shared by the tests and the benchmark; holds input generation only (no selector arithmetic).
Bulk random numbers come from ``synth.c`` (counter-based, so thread count never changes a bit);
this module composes them into the five workloads:

=============  ===  ==  ==  ======  ====  ===  ======  ========  =========
name           B    L   k   V       H     r    logits  hidden/W  codebooks
=============  ===  ==  ==  ======  ====  ===  ======  ========  =========
tiny           1    4   4   1024    64    16   fp32    fp32      fp32
qwen3-8b-b1    1    16  16  151936  4096  64   bf16    bf16      bf16
serving-b64    64   16  16  151936  4096  64   bf16    bf16      bf16
gemma4-31b     32   16  16  262144  5376  128  bf16    bf16      bf16
stress         256  8   32  151936  4096  64   fp32    bf16      bf16
=============  ===  ==  ==  ======  ====  ===  ======  ========  =========

Distributions (every tensor seeded; sequence b of a workload uses seed ``base * 2**20 + b`` for
its logits, hidden rows and anchor; W_sel and the codebooks use the base seed):

* hidden ~ N(0, 1); W_sel ~ N(0, 1/H); pred_cb, succ_cb ~ N(0, 1/r); anchor ~ U{0..V-1}.
* tiny: logits ~ N(0, 3^2), 3 distinct tokens per row get +6.
* qwen3-8b-b1 / serving-b64: logits ~ N(0, 3^2), 8 distinct tokens per row get +U[4, 8].
* gemma4-31b: logits ~ N(0, 2^2), 32 distinct tokens per row get the Zipf(s=1.1)-ranked boost
  8 * i^-1.1 for i = 1..32.
* stress: logits ~ N(0, 0.1^2) in every row. Even rows (global row index b*L+p) stay near-flat;
  odd rows are sharply peaked: one uniform token gets +12. Exact ties are then planted in every
  row by copying values onto tokens outside the row's top k+2: in near-flat rows the value at
  rank 0 (a tie at the top), then in every row the value at rank floor(k/2) (a tie inside the
  top k), then the value at rank k-1 (ranks taken after the earlier copies), so that pair
  straddles the k-th place and the lower id of the two is kept.
* ladder (a parity recipe, not a workload): as stress's base, but even rows carry a planted
  ladder of k-4 tokens at 1 + 0.125*(k-4-j) (j = 0..k-5) whose top two share one value, then a
  cluster of 8 tokens at exactly 1.0 straddling the k-th place; odd rows get one token at +12
  copied onto a second token and 16 further copied pairs.
* Sums are formed in fp32 and rounded once to bf16 (round to nearest even) where the stored dtype
  is bf16. bf16 tensors are numpy ``uint16`` arrays of raw bits.

The LM-head workloads (``LM_CONFIGS``: R rows of hidden state, an [V, H] LM-head weight, k) feed
the fused LM-head top-k pass: W_lm ~ N(0, 9/H), so hidden ~ N(0, 1) rows give logits of spread
about 3; each row then gets 8 distinct target tokens boosted by U[4, 8]: the row adds
(boost / 9) * W_lm[target] (the target's squared norm is about 9), formed in fp32 before the one
rounding to bf16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "synth.c")
LIBRARY = os.path.join(HERE, "libsynth.so")

# stream ids (one per tensor role)
S_LOGITS, S_BOOST_IDS, S_BOOST_VALS, S_HIDDEN, S_WSEL, S_PRED, S_SUCC, S_ANCHOR, S_TIES = range(1, 10)
S_LM_W, S_LM_HIDDEN, S_LM_IDS, S_LM_BOOST = range(10, 14)


def compile_synth(source: str = SOURCE, output: str = LIBRARY) -> str:
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            compile_synth()
        L = ctypes.CDLL(LIBRARY)
        u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.synth_bits.argtypes = [u64, u64, u64]
        L.synth_bits.restype = u64
        L.synth_fill_normal_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
        L.synth_fill_uniform_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
        L.synth_fill_index.argtypes = [u64, u64, u64, i64, i64, vp]
        L.synth_distinct_ids.argtypes = [u64, u64, i64, i64, i64, ctypes.c_int, vp]
        L.synth_f32_to_bf16.argtypes = [vp, i64, vp]
        for f in (L.synth_fill_normal_f32, L.synth_fill_uniform_f32, L.synth_fill_index,
                  L.synth_distinct_ids, L.synth_f32_to_bf16):
            f.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- primitives -------------------------------------------------------------------------------

def normal(seed: int, stream: int, n: int, std: float = 1.0, mean: float = 0.0,
           offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_fill_normal_f32(seed, stream, offset, n, mean, std, _p(out))
    return out


def uniform(seed: int, stream: int, n: int, lo: float, hi: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_fill_uniform_f32(seed, stream, offset, n, lo, hi, _p(out))
    return out


def index(seed: int, stream: int, n: int, n_values: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_fill_index(seed, stream, offset, n, n_values, _p(out))
    return out


def distinct_ids(seed: int, stream: int, nrows: int, n_values: int, m: int,
                 row0: int = 0) -> np.ndarray:
    if m > n_values:
        raise ValueError("m distinct ids need m <= n_values")
    out = np.empty((nrows, m), np.int32)
    lib().synth_distinct_ids(seed, stream, row0, nrows, n_values, m, _p(out))
    return out


def to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().synth_f32_to_bf16(_p(x), x.size, _p(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits (uint16) to float32, for inspection in tests."""
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- workloads --------------------------------------------------------------------------------

@dataclass(frozen=True)
class Spec:
    name: str
    B: int
    L: int
    k: int
    V: int
    H: int
    r: int
    logits_dtype: str  # "f32" | "bf16"
    act_dtype: str     # hidden and W_sel
    cb_dtype: str      # pred_cb and succ_cb
    recipe: str        # "tiny" | "boost8" | "zipf32" | "stress" | "ladder" | "normal"
    seed: int

    @property
    def R(self) -> int:
        return self.B * self.L


CONFIGS = {
    "tiny": Spec("tiny", 1, 4, 4, 1024, 64, 16, "f32", "f32", "f32", "tiny", 1001),
    "qwen3-8b-b1": Spec("qwen3-8b-b1", 1, 16, 16, 151936, 4096, 64, "bf16", "bf16", "bf16",
                        "boost8", 2002),
    "serving-b64": Spec("serving-b64", 64, 16, 16, 151936, 4096, 64, "bf16", "bf16", "bf16",
                        "boost8", 3003),
    "gemma4-31b": Spec("gemma4-31b", 32, 16, 16, 262144, 5376, 128, "bf16", "bf16", "bf16",
                       "zipf32", 4004),
    "stress": Spec("stress", 256, 8, 32, 151936, 4096, 64, "f32", "bf16", "bf16", "stress", 5005),
}
CONFIG_ORDER = ["tiny", "qwen3-8b-b1", "serving-b64", "gemma4-31b", "stress"]


def spec(name: str, **overrides) -> Spec:
    """A named workload, optionally with fields replaced (e.g. a smaller B for a sample)."""
    return replace(CONFIGS[name], **overrides)


@dataclass
class Inputs:
    spec: Spec
    logits: np.ndarray      # [B, L, V] float32 or uint16 (bf16 bits)
    hidden: np.ndarray      # [B, L, H]
    W_sel: np.ndarray       # [H, r]
    pred_cb: np.ndarray     # [V, r]
    succ_cb: np.ndarray     # [V, r]
    anchor_ids: np.ndarray  # [B] int32


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def sequence_seed(base: int, b: int) -> int:
    return base * (1 << 20) + b


def _logit_rows(s: Spec, b: int) -> np.ndarray:
    """fp32 logits [L, V] of sequence b, before rounding to the stored dtype."""
    sb = sequence_seed(s.seed, b)
    L, V, k = s.L, s.V, s.k
    if s.recipe == "tiny":
        x = normal(sb, S_LOGITS, L * V, std=3.0).reshape(L, V)
        ids = distinct_ids(sb, S_BOOST_IDS, L, V, 3)
        for p in range(L):
            x[p, ids[p]] += np.float32(6.0)
    elif s.recipe == "boost8":
        x = normal(sb, S_LOGITS, L * V, std=3.0).reshape(L, V)
        ids = distinct_ids(sb, S_BOOST_IDS, L, V, 8)
        val = uniform(sb, S_BOOST_VALS, L * 8, 4.0, 8.0).reshape(L, 8)
        for p in range(L):
            x[p, ids[p]] += val[p]
    elif s.recipe == "zipf32":
        x = normal(sb, S_LOGITS, L * V, std=2.0).reshape(L, V)
        ids = distinct_ids(sb, S_BOOST_IDS, L, V, 32)
        boost = (8.0 * np.arange(1, 33, dtype=np.float64) ** -1.1).astype(np.float32)
        for p in range(L):
            x[p, ids[p]] += boost
    elif s.recipe == "stress":
        x = normal(sb, S_LOGITS, L * V, std=0.1).reshape(L, V)
        peak = index(sb, S_BOOST_IDS, L, V)
        draws = index(sb, S_TIES, L * 64, V).reshape(L, 64)
        for p in range(L):
            flat = (b * L + p) % 2 == 0
            if not flat:
                x[p, peak[p]] += np.float32(12.0)
            _plant_ties(x[p], k, flat, draws[p])
    elif s.recipe == "ladder":
        x = normal(sb, S_LOGITS, L * V, std=0.1).reshape(L, V)
        m = k + 4
        ids = distinct_ids(sb, S_TIES, L, V, max(m, 34))
        for p in range(L):
            row = ids[p]
            if (b * L + p) % 2 == 0:
                n_ladder = max(k - 4, 2)
                ladder = (1.0 + 0.125 * (n_ladder - np.arange(n_ladder))).astype(np.float32)
                ladder[1] = ladder[0]
                x[p, row[:n_ladder]] = ladder
                x[p, row[n_ladder:n_ladder + 8]] = np.float32(1.0)
            else:
                x[p, row[0]] += np.float32(12.0)
                x[p, row[1]] = x[p, row[0]]
                for t in range(16):
                    x[p, row[2 + 2 * t + 1]] = x[p, row[2 + 2 * t]]
    elif s.recipe == "normal":
        x = normal(sb, S_LOGITS, L * V, std=3.0).reshape(L, V)
    else:
        raise ValueError(f"unknown recipe {s.recipe}")
    return x


def _plant_ties(row: np.ndarray, k: int, flat: bool, draws: np.ndarray) -> None:
    """Copy values of the row's leading tokens onto tokens outside its top k+2 (in place): rank 0
    (near-flat rows only), then rank floor(k/2), then rank k-1, each rank taken after the earlier
    copies. Ranks follow the stored values (larger first, lower id first among equal ones); the
    targets come from `draws` (seeded ids), skipping tokens already among the leaders."""
    V = row.size
    m = min(k + 2, V)
    if m < 2:
        return
    lead = np.argpartition(-row, m - 1)[:m]
    top = sorted(((float(row[i]), int(i)) for i in lead), key=lambda t: (-t[0], t[1]))
    used = {i for _, i in top}
    it = iter(draws.tolist())

    def target() -> int | None:
        for t in it:
            if t not in used:
                used.add(t)
                return t
        for t in range(V):  # (only for tiny rows: the seeded draws ran out)
            if t not in used:
                used.add(t)
                return t
        return None

    for rank in ([0] if flat else []) + [k // 2, k - 1]:
        if rank >= len(top):
            continue
        t = target()
        if t is None:
            return
        v = top[rank][0]
        row[t] = np.float32(v)
        top.append((v, t))
        top.sort(key=lambda e: (-e[0], e[1]))


def make_inputs(s: Spec | str, **overrides) -> Inputs:
    """Generate the workload ``s`` (a Spec or a config name) on the host."""
    if isinstance(s, str):
        s = spec(s, **overrides)
    elif overrides:
        s = replace(s, **overrides)
    B, L, V, H, r = s.B, s.L, s.V, s.H, s.r
    ldt = np.uint16 if s.logits_dtype == "bf16" else np.float32
    logits = np.empty((B, L, V), ldt)
    hidden = np.empty((B, L, H), np.uint16 if s.act_dtype == "bf16" else np.float32)
    anchor = np.empty((B,), np.int32)
    for b in range(B):
        logits[b] = _store(_logit_rows(s, b), s.logits_dtype)
        sb = sequence_seed(s.seed, b)
        hidden[b] = _store(normal(sb, S_HIDDEN, L * H).reshape(L, H), s.act_dtype)
        anchor[b] = index(sb, S_ANCHOR, 1, V)[0]
    W_sel = _store(normal(s.seed, S_WSEL, H * r, std=1.0 / np.sqrt(H)).reshape(H, r), s.act_dtype)
    pred = _store(normal(s.seed, S_PRED, V * r, std=1.0 / np.sqrt(r)).reshape(V, r), s.cb_dtype)
    succ = _store(normal(s.seed, S_SUCC, V * r, std=1.0 / np.sqrt(r)).reshape(V, r), s.cb_dtype)
    return Inputs(s, logits, hidden, W_sel, pred, succ, anchor)


def as_torch(a: np.ndarray, device=None):
    """numpy float32 / uint16 (bf16 bits) / int32 -> torch tensor (bf16 for uint16)."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device) if device is not None else t


def from_torch(t) -> np.ndarray:
    """torch tensor -> numpy (bf16 becomes uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ---- LM-head workloads ------------------------------------------------------------------------

@dataclass(frozen=True)
class LmSpec:
    name: str
    R: int
    H: int
    V: int
    k: int
    seed: int


LM_CONFIGS = {
    "lmhead-qwen3-8b-b1": LmSpec("lmhead-qwen3-8b-b1", 16, 4096, 151936, 16, 6006),
    "lmhead-serving-b64": LmSpec("lmhead-serving-b64", 1024, 4096, 151936, 16, 7007),
}


def lmhead_inputs(R: int, H: int, V: int, seed: int, targets: int = 8):
    """hidden [R, H] and W_lm [V, H], both bf16 bits (see the module notes)."""
    sw = 3.0 / np.sqrt(H)
    W = normal(seed, S_LM_W, V * H, std=sw).reshape(V, H)
    z = normal(seed, S_LM_HIDDEN, R * H).reshape(R, H)
    m = min(targets, V)
    if m > 0:
        ids = distinct_ids(seed, S_LM_IDS, R, V, m)
        val = uniform(seed, S_LM_BOOST, R * m, 4.0, 8.0).reshape(R, m)
        scale = np.float32(1.0 / (H * sw * sw))
        for i in range(R):
            for j in range(m):
                z[i] += (val[i, j] * scale) * W[ids[i, j]]
    return to_bf16(z), to_bf16(W)
