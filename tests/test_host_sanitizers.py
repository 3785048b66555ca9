"""The oracle and the input generator under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; both are plain C built with gcc, no GPU code is involved).

Each C source is built with -fsanitize=address,undefined into a temporary directory. A child
Python process, with the ASan runtime preloaded (the interpreter itself is not instrumented),
runs every oracle pin against the sanitized oracle and generates workloads with the sanitized
generator, comparing them bit for bit with the regular build. Any sanitizer report, or a
difference, fails the test.
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _gcc_runtime(name: str) -> str:
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                         check=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else ""


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    asan = _gcc_runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's ASan runtime is not installed")
    d = tmp_path_factory.mktemp("sanitized")
    ora = os.path.join(d, "liboracle_san.so")
    syn = os.path.join(d, "libsynth_san.so")
    subprocess.run(["gcc", *SAN, "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-o", ora, oracle.SOURCE, "-lm"], check=True)
    subprocess.run(["gcc", *SAN, "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", syn, synth.SOURCE, "-lm"], check=True)
    return asan, ora, syn


CHILD = textwrap.dedent("""
    import ctypes, sys
    import numpy as np
    sys.path[:0] = [{root!r}, {tests!r}]
    import oracle, synth
    from oracle_pins import PINS
    o = oracle.Oracle({ora!r})
    for pin in PINS:
        pin(o)
    print("pins", len(PINS), flush=True)
    specs = [synth.spec("tiny"), synth.spec("qwen3-8b-b1", L=2, V=20011),
             synth.spec("gemma4-31b", B=1, L=2, V=30000, H=512),
             synth.spec("stress", B=1, L=4, V=5000, H=256), synth.spec("stress", B=1, L=3,
             recipe="ladder", V=3000, H=64)]
    plain = [synth.make_inputs(s) for s in specs]
    synth._lib = None
    synth.LIBRARY = {syn!r}
    for s, a in zip(specs, plain):
        b = synth.make_inputs(s)
        for f in ("logits", "hidden", "W_sel", "pred_cb", "succ_cb", "anchor_ids"):
            assert np.array_equal(getattr(a, f), getattr(b, f)), (s.name, f)
        r = o.select(b.logits, b.hidden, b.W_sel, b.pred_cb, b.succ_cb, b.anchor_ids, s.k)
        assert np.isfinite(r.edges).all()
    hb, wb = synth.lmhead_inputs(5, 64, 300, 3)
    o.lmhead_topk(hb, wb, 4)
    print("generator ok", flush=True)
""")


def test_oracle_and_generator_under_sanitizers(sanitized):
    asan, ora, syn = sanitized
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=24"
    env["OMP_NUM_THREADS"] = "2"
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), ora=ora, syn=syn)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    assert "generator ok" in r.stdout
