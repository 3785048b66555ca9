"""Benchmark of the DFlash 2 candidate selector on one MI355X.

A step is one dflash2_select call: top-k + logsumexp, gate, lattice and walk over one batch of
synthetic logits/hidden rows already resident in HBM. Every timed loop runs its W warm-up steps
and keeps warming (untimed) until at least WARM_SECONDS have passed: the GPU's clocks take tens
of milliseconds of load to settle, and a selector in serving runs back to back. Logits and hidden rows rotate through a
pool of copies larger than 1 GiB (over twice the 256 MB Infinity Cache), so every step streams
its logits from HBM. The weights (W_sel, codebooks) are one copy, as in serving.

Prints one JSON line:
  value        selector positions/s = B*L*steps / elapsed (the default workload: serving-b64)
  roofline     K1 (the top-k/logsumexp pass, the dominant kernel): algorithmic bytes per launch
               (R*V*elem + R*k*8 + R*4) / mean K1 launch time (HIP events around graph replays of
               K1-only launches on the launch stream; the eager loop's time, which also holds the
               dispatch gap between launches, is given beside it), against the MI355X HBM peak of
               8 TB/s; `traffic`
               comes from committed rocprofv3 counter readings when they match the current kernel
  cpu_baseline the fp64 C oracle on the host, on the same workload: row-parallel over the host's
               cores (value, cores) and single-threaded (single_thread), with the CPU model
  per_config   end-to-end latency and K1 bandwidth of every workload (eager launches; `graph`:
               the same calls captured in a HIP graph and replayed, the GPU side without the
               host's per-call launch cost)
  extras       the default workload with the walk's sampling and p_min modes, its gate product
               alone (dflash2_gate: flops against the bf16 matrix-core peak, bytes against HBM),
               the grouped
               dynamic depthwise convolution at the serving block shape, and the LM-head product
               with the top-k pass folded in (16 rows, V = 151936, H = 4096), against its HBM
               roofline, beside a library product followed by the top-k pass
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selector positions/sec and top-k pass HBM GB/s (% of peak) at V=151936, L=16, k=16"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix cores
POOL_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_lse_traffic.json")
# the sources the streaming top-k kernel is compiled from (the traffic readings name their hash)
K1_SOURCES = [os.path.join(ROOT, "dflash2_draft_candidate_amd", "csrc", f)
              for f in ("topk_lse.hip", "row_slices.h", "device_common.h", "gate_tile.h")]
K1_KERNEL = "topk_lse_kernel"
COPY_KERNEL = "copyBuffer"  # the HIP runtime's device-to-device copy kernel
COPY_REPS = 5
WARM_SECONDS = 0.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def k1_bytes(s) -> int:
    elem = 2 if s.logits_dtype == "bf16" else 4
    return s.R * (s.V * elem + s.k * 8 + 4)


def source_hash(paths: list[str]) -> str:
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


class Workload:
    """Device-resident inputs for one workload, with a rotating pool of logits/hidden copies."""

    def __init__(self, name: str, device: str):
        import synth
        import torch
        t0 = time.time()
        self.x = synth.make_inputs(name)
        self.s = self.x.spec
        t1 = time.time()
        logits = synth.as_torch(self.x.logits, device)
        hidden = synth.as_torch(self.x.hidden, device)
        per = logits.numel() * logits.element_size() + hidden.numel() * hidden.element_size()
        n = min(512, max(1, -(-POOL_BYTES // per)))
        self.logits = [logits] + [logits.clone() for _ in range(n - 1)]
        self.hidden = [hidden] + [hidden.clone() for _ in range(n - 1)]
        self.W = synth.as_torch(self.x.W_sel, device)
        self.pred = synth.as_torch(self.x.pred_cb, device)
        self.succ = synth.as_torch(self.x.succ_cb, device)
        self.anchor = synth.as_torch(self.x.anchor_ids, device)
        s = self.s
        self.out = (torch.empty((s.B, s.L, s.k), dtype=torch.int32, device=device),
                    torch.empty((s.B, s.L, s.k), dtype=torch.float32, device=device),
                    torch.empty((s.B, s.L, s.k, s.k), dtype=torch.float32, device=device),
                    torch.empty((s.B, s.L), dtype=torch.int32, device=device))
        import dflash2_draft_candidate_amd as d2
        self.ws = torch.empty(max(16, d2.workspace_bytes(s.B, s.L, s.V, s.H, s.r, s.k)),
                              dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        log(f"[bench] {name}: generated in {t1 - t0:.1f}s, pool of {n} logits/hidden copies")

    def step(self, i: int):
        import dflash2_draft_candidate_amd as d2
        j = i % len(self.logits)
        d2.select(self.logits[j], self.hidden[j], self.W, self.pred, self.succ, self.anchor,
                  self.s.k, out=self.out, workspace=self.ws)

    def k1_step(self, i: int, ids, unary, lse, ws):
        import ctypes
        import dflash2_draft_candidate_amd as d2
        import torch
        j = i % len(self.logits)
        s = self.s
        lg = self.logits[j]
        rc = d2.library().dflash2_topk_lse(
            ctypes.c_void_p(lg.data_ptr()), d2._dtype(lg), s.R, s.V, s.k,
            ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(unary.data_ptr()),
            ctypes.c_void_p(lse.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"dflash2_topk_lse failed with status {rc}")


def time_loop(fn, steps: int, warmup: int, warm_seconds: float = WARM_SECONDS,
              stats: dict | None = None) -> float:
    """Mean milliseconds per call of fn(i), HIP events on the current stream, after `warmup`
    untimed calls and as many more as fill warm_seconds. With `stats`, an event is also recorded
    between consecutive calls and the per-call median, p10 and p90 go into it (the event records
    are enqueued between launches, so the mean of the per-call times is the same region)."""
    import torch
    t0 = time.time()
    i = 0
    while i < warmup or time.time() - t0 < warm_seconds:
        fn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    n_ev = steps + 1 if stats is not None else 2
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev[0].record()
    for j in range(steps):
        fn(i + j)
        if stats is not None:
            ev[j + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[-1])
    if stats is not None:
        per = sorted(ev[j].elapsed_time(ev[j + 1]) for j in range(steps))
        q = lambda f: per[min(steps - 1, int(round(f * (steps - 1))))]
        stats.update({"median_us": round(q(0.5) * 1e3, 2), "p10_us": round(q(0.1) * 1e3, 2),
                      "p90_us": round(q(0.9) * 1e3, 2)})
    return total / steps


def graph_loop(fn, n: int, replays: int, warm_seconds: float = WARM_SECONDS) -> float:
    """Mean milliseconds per call of fn(j) when calls j = 0 .. n-1 are captured once in a HIP
    graph and the graph is replayed `replays` times (HIP events around the replays, after
    warm_seconds of untimed replays): the GPU side of the step without the host's per-call
    launch cost, which bounds the eager loop at small sizes."""
    import torch
    for j in range(n):
        fn(j)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            fn(j)
    t0 = time.time()
    while time.time() - t0 < warm_seconds:
        g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * n)


GRAPH_CALLS = 32  # calls per captured graph (over distinct pool copies)


def measure(name: str, device: str, steps: int, warmup: int) -> dict:
    import torch
    w = Workload(name, device)
    s = w.s
    e2e_stats, k1_stats = {}, {}
    e2e_ms = time_loop(w.step, steps, warmup, stats=e2e_stats)
    ids = torch.empty((s.R, s.k), dtype=torch.int32, device=device)
    unary = torch.empty((s.R, s.k), dtype=torch.float32, device=device)
    lse = torch.empty((s.R,), dtype=torch.float32, device=device)
    import dflash2_draft_candidate_amd as d2
    from dflash2_draft_candidate_amd import BF16, F32
    wsb = d2.library().dflash2_topk_lse_workspace_bytes(s.R, s.V, s.k,
                                                        BF16 if s.logits_dtype == "bf16" else F32)
    ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=device)
    k1_ms = time_loop(lambda i: w.k1_step(i, ids, unary, lse, ws), steps, warmup,
                      stats=k1_stats)
    gbs = k1_bytes(s) / (k1_ms * 1e-3) / 1e9
    n_graph = min(GRAPH_CALLS, len(w.logits))
    replays = max(1, steps // n_graph)
    e2e_graph_ms = graph_loop(w.step, n_graph, replays)
    k1_graph_ms = graph_loop(lambda i: w.k1_step(i, ids, unary, lse, ws), n_graph, replays)
    gbs_graph = k1_bytes(s) / (k1_graph_ms * 1e-3) / 1e9
    res = {"B": s.B, "L": s.L, "k": s.k, "V": s.V, "H": s.H, "r": s.r,
           "logits": s.logits_dtype, "e2e_us": round(e2e_ms * 1e3, 2),
           "positions_per_s": round(s.R / (e2e_ms * 1e-3), 1), "k1_us": round(k1_ms * 1e3, 2),
           "k1_gbs": round(gbs, 1), "k1_frac": round(gbs / PEAK_HBM_GBS, 4),
           "e2e_us_per_step": e2e_stats, "k1_us_per_step": k1_stats,
           "graph": {"calls_per_graph": n_graph, "replays": replays,
                     "e2e_us": round(e2e_graph_ms * 1e3, 2),
                     "positions_per_s": round(s.R / (e2e_graph_ms * 1e-3), 1),
                     "k1_us": round(k1_graph_ms * 1e3, 2), "k1_gbs": round(gbs_graph, 1),
                     "k1_frac": round(gbs_graph / PEAK_HBM_GBS, 4)}}
    res["_workload"] = w
    return res


def measure_modes(w, steps: int, warmup: int) -> dict:
    """The selector with the walk's further modes on a workload's inputs: sampling at T = 1
    (staged lattice + walk kernels) and the greedy p_min stop (fused)."""
    import torch
    import dflash2_draft_candidate_amd as d2
    s = w.s
    dev = w.W.device
    u = torch.rand((s.B, s.L), generator=torch.Generator().manual_seed(7)).to(dev)
    out = tuple(torch.empty_like(t) for t in w.out) + (torch.empty((s.B,), dtype=torch.int32,
                                                                   device=dev),)
    res = {}
    for name, T, p_min in (("sample_T1", 1.0, 0.0), ("greedy_pmin0.3", 0.0, 0.3)):
        def step(i, T=T, p_min=p_min):
            j = i % len(w.logits)
            d2.select_ex(w.logits[j], w.hidden[j], w.W, w.pred, w.succ, w.anchor, s.k, T,
                         u if T > 0 else None, p_min, out=out, workspace=w.ws)
        ms = time_loop(step, steps, warmup)
        res[name] = {"e2e_us": round(ms * 1e3, 2), "positions_per_s": round(s.R / (ms * 1e-3), 1)}
    return res


def measure_dynconv(device: str, steps: int, warmup: int) -> dict:
    """The grouped dynamic depthwise convolution at the serving block shape: 64 blocks of the
    verified token + 16 draft rows, hidden size 4096, 2 taps, groups of 16, bf16."""
    import torch
    import dflash2_draft_candidate_amd as d2
    nb, T, C, K, G = 64, 17, 4096, 2, 16
    g = torch.Generator().manual_seed(11)
    x = torch.randn((nb, T, C), generator=g).to(torch.bfloat16).to(device)
    base = (0.5 * torch.randn((K, C), generator=g)).to(torch.bfloat16).to(device)
    dyn = (0.1 * torch.randn((nb, T, K, C // G), generator=g)).to(torch.bfloat16).to(device)
    y = torch.empty_like(x)
    # the kernel lasts a few microseconds, less than a Python call: time it inside a HIP graph
    # of `reps` launches, replayed, so the host's launch cost stays out of the measurement
    reps = 50
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        d2.dynconv(x, base, dyn, G, out=y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            d2.dynconv(x, base, dyn, G, out=y)
    ms = time_loop(lambda i: graph.replay(), max(1, steps // 10), warmup) / reps
    nbytes = 2 * (2 * nb * T * C + nb * T * K * (C // G) + K * C)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"shape": {"n_blocks": nb, "T": T, "C": C, "K": K, "group": G, "dtype": "bf16"},
            "launch_us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def measure_gate(w, steps: int, warmup: int) -> dict:
    """The stand-alone gate product g = hidden . W_sel (dflash2_gate) on the workload's rows:
    launch time over a rotating pool of hidden copies, its rate in flops (2 R H r) against the
    dense bf16 matrix-core peak and in algorithmic bytes (hidden, W_sel, the fp32 g) against HBM;
    with H r / (H + r) flops per byte it is bound by HBM."""
    import ctypes
    import torch
    import dflash2_draft_candidate_amd as d2
    s = w.s
    R, H, r = s.R, s.H, s.r
    hid = [h.reshape(R, H) for h in w.hidden]
    g = torch.empty((R, r), dtype=torch.float32, device=hid[0].device)
    lib = d2.library()
    ws = torch.empty(max(16, lib.dflash2_gate_workspace_bytes(R, H, r)), dtype=torch.uint8,
                     device=hid[0].device)
    dt = d2._dtype(hid[0])

    def step(i):
        rc = lib.dflash2_gate(ctypes.c_void_p(hid[i % len(hid)].data_ptr()),
                              ctypes.c_void_p(w.W.data_ptr()), dt, R, H, r,
                              ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                              ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"dflash2_gate failed with status {rc}")

    ms = time_loop(step, steps, warmup)
    graph_ms = graph_loop(step, min(GRAPH_CALLS, len(hid)), max(1, steps // GRAPH_CALLS))
    el = hid[0].element_size()
    flops = 2.0 * R * H * r
    nbytes = R * H * el + H * r * el + R * r * 4
    return {"shape": {"R": R, "H": H, "r": r, "dtype": s.act_dtype},
            "launch_us": round(ms * 1e3, 2), "graph_launch_us": round(graph_ms * 1e3, 2),
            "tflops": round(flops / (graph_ms * 1e-3) / 1e12, 2),
            "frac_mfma_bf16": round(flops / (graph_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "algorithmic_bytes": nbytes, "gbs": round(nbytes / (graph_ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "bound": "hbm"}


def measure_lmhead(device: str, steps: int, warmup: int) -> dict:
    """The LM-head product with the top-k pass folded into it (dflash2_lmhead_topk) at the
    lmhead-qwen3-8b-b1 shape: 16 rows of hidden state, H = 4096, V = 151936, k = 16, bf16. Its
    roofline is HBM: the [V, H] weight is read once. For context, the same result from a library
    product that writes bf16 logits (torch.matmul) followed by the top-k pass."""
    import torch
    import dflash2_draft_candidate_amd as d2
    import synth
    s = synth.LM_CONFIGS["lmhead-qwen3-8b-b1"]
    hb, wb = synth.lmhead_inputs(s.R, s.H, s.V, s.seed)
    h, w = synth.as_torch(hb, device), synth.as_torch(wb, device)
    del hb, wb
    ms = time_loop(lambda i: d2.lmhead_topk(h, w, s.k), max(4, steps // 4), warmup)
    nbytes = 2 * (s.V * s.H + s.R * s.H) + s.R * (8 * s.k + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    ms_unfused = time_loop(lambda i: d2.topk_lse(torch.matmul(h, w.t()), s.k), max(4, steps // 4),
                           warmup)
    del h, w
    torch.cuda.empty_cache()
    return {"shape": {"workload": s.name, "R": s.R, "H": s.H, "V": s.V, "k": s.k,
                      "dtype": "bf16"},
            "us": round(ms * 1e3, 2), "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "tflops": round(2.0 * s.R * s.H * s.V / (ms * 1e-3) / 1e12, 1),
            "unfused_matmul_plus_topk_us": round(ms_unfused * 1e3, 2)}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads(cap: int) -> int:
    """Threads for the row-parallel oracle: the cores this process may run on, no more than
    OMP_NUM_THREADS when that is set (the host's share of cores per GPU), nor than `cap`."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, min(n, cap))


def cpu_baseline(name: str, seconds_1: float = 8.0, seconds_n: float = 6.0,
                 max_passes: int = 512) -> dict:
    """The oracle (fp64 C) on the host over whole passes of the workload: single-threaded, then
    row-parallel (the sequences split into contiguous groups, one oracle call per group on a pool
    of threads; ctypes releases the GIL during each call, and sequences are independent, so the
    outputs are those of the single-threaded pass, which is checked)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    import synth
    x = synth.make_inputs(name)
    o = oracle.default()
    B, R = x.spec.B, x.spec.R

    def run(b0, b1):
        return o.select(x.logits[b0:b1], x.hidden[b0:b1], x.W_sel, x.pred_cb, x.succ_cb,
                        x.anchor_ids[b0:b1], x.spec.k)

    passes1, el1, ref = 0, 0.0, None
    while passes1 < max_passes and (passes1 == 0 or el1 < seconds_1):
        t0 = time.perf_counter()
        ref = run(0, B)
        el1 += time.perf_counter() - t0
        passes1 += 1
    n = host_threads(B)
    bounds = [(B * i // n, B * (i + 1) // n) for i in range(n)]
    passesn, eln, parts = 0, 0.0, None
    with ThreadPoolExecutor(max_workers=n) as ex:
        while passesn < max_passes and (passesn == 0 or eln < seconds_n):
            t0 = time.perf_counter()
            parts = list(ex.map(lambda bb: run(*bb), bounds))
            eln += time.perf_counter() - t0
            passesn += 1
    got = np.concatenate([p.path for p in parts])
    if not np.array_equal(got, ref.path) or \
            not np.array_equal(np.concatenate([p.cand_ids for p in parts]), ref.cand_ids):
        raise RuntimeError("row-parallel oracle differs from the single-threaded pass")
    v1, vn = R * passes1 / el1, R * passesn / eln
    return {"value": round(vn, 1), "unit": "positions/s", "cores": n, "kind": "oracle",
            "sample": f"{passesn} full pass(es) of the {name} workload ({R} positions each) in "
                      f"{eln:.1f} s, {n} threads, row-parallel fp64 C (sequences split over the "
                      f"threads)",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "single_thread": {"value": round(v1, 1), "unit": "positions/s", "cores": 1,
                              "sample": f"{passes1} full pass(es) in {el1:.1f} s"}}


def committed_traffic() -> dict | None:
    """HBM bytes per K1 launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE readings, if they
    were taken on the current K1 source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("k1_source_sha256_16") != source_hash(K1_SOURCES):
        return None
    return t


def _kernel_name(n: str) -> str:
    n = n.replace("void ", "").replace("dflash2::(anonymous namespace)::", "")
    return n.split("(")[0]


def _counter_rows(path: str, counter: str):
    """(kernel name, value) of every dispatch in a rocprofv3 counter_collection.csv, in dispatch
    order."""
    import csv
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]


def summarize(a: list[str]):
    """Write a profiles/ summary from rocprofv3 output (runs on the host, no GPU)."""
    import csv
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    if a[0] == "trace":
        stats, out_md, cmd = a[1], a[2], a[3]
        lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "",
                 "Command (from the repository root on a one-GPU MI355X box):", "",
                 f"    {cmd}", "",
                 "| kernel | calls | avg us | min us | max us | share of GPU time |",
                 "|---|---|---|---|---|---|"]
        for r in csv.DictReader(open(stats)):
            lines.append(f"| `{_kernel_name(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
        open(out_md, "w").write("\n".join(lines) + "\n")
        print(out_md)
        return
    if a[0] == "traffic":
        import synth
        fetch_csv, write_csv, workload, cmd = a[1], a[2], a[3], a[4]
        reads = {}
        for which, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"),
                                     ("write", write_csv, "WRITE_SIZE")):
            rows = _counter_rows(path, counter)
            k1 = [v for n, v in rows if K1_KERNEL in n]
            # the calibration copies are the last COPY_REPS copies (earlier ones build the pool)
            cp = [v for n, v in rows if COPY_KERNEL in n][-COPY_REPS:]
            if not k1 or not cp:
                raise SystemExit(f"{path}: no {K1_KERNEL} or {COPY_KERNEL} dispatches")
            reads[which] = (sum(k1) / len(k1), sum(cp) / len(cp), len(k1), len(cp))
        copy_bytes = int(cmd.split("--copy-mib")[1].split()[0]) << 20
        f_k1, f_cp, n1, n2 = reads["fetch"]
        w_k1, w_cp, _, _ = reads["write"]
        f_factor = f_cp * 1024 / copy_bytes  # counter bytes per byte really read
        w_factor = w_cp * 1024 / copy_bytes
        fetch_b = f_k1 * 1024 / f_factor
        write_b = w_k1 * 1024 / w_factor
        s = synth.spec(workload)
        t = {"kernel": K1_KERNEL, "workload": workload,
             "k1_source_sha256_16": source_hash(K1_SOURCES),
             "bytes_per_launch": int(round(fetch_b + write_b)),
             "fetch_bytes_per_launch": int(round(fetch_b)),
             "write_bytes_per_launch": int(round(write_b)),
             "algorithmic_bytes_per_launch": k1_bytes(s),
             "raw_fetch_kib_per_launch": round(f_k1, 1), "raw_write_kib_per_launch": round(w_k1, 1),
             "copy_bytes": copy_bytes, "copy_fetch_kib": round(f_cp, 1),
             "copy_write_kib": round(w_cp, 1), "fetch_factor": round(f_factor, 4),
             "write_factor": round(w_factor, 4), "k1_dispatches": n1, "copy_dispatches": n2,
             "command": cmd}
        json.dump(t, open(TRAFFIC_FILE, "w"), indent=1)
        md = os.path.join(ROOT, "profiles", f"topk_lse_{workload}_traffic.md")
        open(md, "w").write(
            f"# HBM traffic of {K1_KERNEL} on {workload}\n\n"
            "Two rocprofv3 counter passes over the same command (FETCH_SIZE, then WRITE_SIZE), "
            "from the repository root on a one-GPU MI355X box:\n\n"
            f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_FETCH_SIZE -o k1 -- {cmd}\n"
            f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_WRITE_SIZE -o k1 -- {cmd}\n\n"
            f"Calibration: the runtime's copy kernel moving {copy_bytes} bytes reads "
            f"{f_cp:.1f} KiB of FETCH_SIZE and {w_cp:.1f} KiB of WRITE_SIZE per dispatch: "
            f"factors {f_factor:.4f} (fetch) and {w_factor:.4f} (write) counter bytes per byte.\n\n"
            f"| per K1 launch | bytes |\n|---|---|\n"
            f"| FETCH_SIZE raw | {f_k1 * 1024:.0f} |\n| WRITE_SIZE raw | {w_k1 * 1024:.0f} |\n"
            f"| fetch (calibrated) | {fetch_b:.0f} |\n| write (calibrated) | {write_b:.0f} |\n"
            f"| traffic (calibrated) | {fetch_b + write_b:.0f} |\n"
            f"| algorithmic | {k1_bytes(s)} |\n"
            f"| traffic / algorithmic | {(fetch_b + write_b) / k1_bytes(s):.4f} |\n")
        print(TRAFFIC_FILE, md)
        return
    if a[0] == "counters":
        import synth
        csv_paths, out_md, workload, cmd = a[1].split(","), a[2], a[3], a[4]
        s = synth.spec(workload)
        rows = []
        for path in csv_paths:
            rows += list(csv.DictReader(open(path)))
        per = {}   # kernel -> counter -> values (one per dispatch)
        for r in rows:
            k = _kernel_name(r["Kernel_Name"])
            if "copyBuffer" in k or "fill" in k.lower() or "elementwise" in k.lower():
                continue
            per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
        names = sorted({c for v in per.values() for c in v})
        lines = [f"# Counters: {os.path.basename(out_md)[:-3]}", "",
                 "rocprofv3 counter passes, one run per pass (from the repository root on a "
                 "one-GPU MI355X box):", ""]
        lines += [f"    {c}" for c in cmd.split(" ;; ")]
        lines += ["", f"Workload {workload}: R = {s.R} rows of V = {s.V} ({s.logits_dtype}).",
                  "Values are means per dispatch over the profiled launches; SQ instruction "
                  "counts are wave instructions summed over the chip, SQ_ACTIVE_INST_VALU and "
                  "SQ_VALU_MFMA_BUSY_CYCLES are summed over the SIMDs.", "",
                  "| kernel | " + " | ".join(names) + " |",
                  "|---|" + "---|" * len(names)]
        for k, cs in sorted(per.items()):
            vals = [f"{sum(cs[n]) / len(cs[n]):.4g}" if n in cs else "" for n in names]
            lines.append(f"| `{k}` | " + " | ".join(vals) + " |")
        elems = s.R * s.V
        derived = []
        for k, cs in sorted(per.items()):
            m = lambda n: sum(cs[n]) / len(cs[n]) if n in cs else None
            # GRBM_GUI_ACTIVE is read on each of the 8 XCDs and summed: the dispatch's busy
            # cycles are an eighth of it
            busy = m("GRBM_GUI_ACTIVE") / 8 if m("GRBM_GUI_ACTIVE") else None
            if busy:
                derived.append(f"| `{k}` | busy cycles (GRBM_GUI_ACTIVE / 8 XCDs) | {busy:.4g} |")
            if busy and m("SQ_ACTIVE_INST_VALU"):
                derived.append(f"| `{k}` | VALU busy (SQ_ACTIVE_INST_VALU x 4 / 1024 SIMDs / "
                               f"busy cycles) | {m('SQ_ACTIVE_INST_VALU') * 4 / 1024 / busy:.3f} |")
            if busy and m("SQ_WAVE_CYCLES"):
                derived.append(f"| `{k}` | mean resident waves per CU (SQ_WAVE_CYCLES x 4 / "
                               f"busy cycles / 256 CUs) | "
                               f"{m('SQ_WAVE_CYCLES') * 4 / busy / 256:.2f} |")
            if busy and m("SQ_VALU_MFMA_BUSY_CYCLES"):
                derived.append(f"| `{k}` | MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / "
                               f"busy cycles) | "
                               f"{m('SQ_VALU_MFMA_BUSY_CYCLES') / busy / 1024:.4f} |")
            if m("SQ_LDS_IDX_ACTIVE") and m("SQ_LDS_BANK_CONFLICT") is not None:
                derived.append(f"| `{k}` | LDS bank-conflict cycles per LDS-active cycle | "
                               f"{m('SQ_LDS_BANK_CONFLICT') / m('SQ_LDS_IDX_ACTIVE'):.4f} |")
            if ("topk_lse_kernel" in k or "topk_small_kernel" in k) and m("SQ_INSTS_VALU"):
                derived.append(f"| `{k}` | VALU instructions per element | "
                               f"{m('SQ_INSTS_VALU') * 64 / elems:.3f} |")
                if m("SQ_INSTS_VALU_TRANS_F32"):
                    derived.append(f"| `{k}` | transcendental instructions per element | "
                                   f"{m('SQ_INSTS_VALU_TRANS_F32') * 64 / elems:.3f} |")
                if m("SQ_ACTIVE_INST_VALU"):
                    derived.append(f"| `{k}` | VALU issue quad-cycles per VALU instruction | "
                                   f"{m('SQ_ACTIVE_INST_VALU') / m('SQ_INSTS_VALU'):.3f} |")
            if m("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
                derived.append(f"| `{k}` | bf16 MFMA flops per dispatch (MOPS x 512) | "
                               f"{m('SQ_INSTS_VALU_MFMA_MOPS_BF16') * 512:.4g} |")
            if m("TCC_HIT_sum") is not None and m("TCC_MISS_sum"):
                h, mi = m("TCC_HIT_sum"), m("TCC_MISS_sum")
                derived.append(f"| `{k}` | L2 hit rate | {h / (h + mi):.3f} |")
        if derived:
            lines += ["", "| kernel | derived | value |", "|---|---|---|"] + derived
        open(out_md, "w").write("\n".join(lines) + "\n")
        print(out_md)
        return
    raise SystemExit(f"unknown summary kind {a[0]}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="serving-b64")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--k1-only", action="store_true",
                    help="only loop K1 launches (for counter collection), no JSON")
    ap.add_argument("--select-only", action="store_true",
                    help="only loop selector calls (for counter collection), no JSON")
    ap.add_argument("--lmhead-only", action="store_true",
                    help="only loop LM-head top-k calls at lmhead-qwen3-8b-b1 (for profiling), "
                         "no JSON")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="with --k1-only: also run device-to-device copies of this many MiB, the "
                         "calibration for the HBM byte counters")
    ap.add_argument("--summarize", nargs="+", metavar="ARG",
                    help="no GPU: 'trace STATS_CSV OUT_MD CMD', 'traffic FETCH_CSV WRITE_CSV "
                         "WORKLOAD CMD' or 'counters CSV[,CSV...] OUT_MD WORKLOAD CMDS' writes a "
                         "profiles/ summary from rocprofv3 output (CMDS: commands joined by ' ;; ')")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each sequence is "
              "independent; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import dflash2_draft_candidate_amd  # noqa: F401  fails loudly if the library is not built
    import synth
    device = "cuda:0"
    torch.cuda.set_device(0)

    if args.select_only:
        w = Workload(args.workload, device)
        # (no time-based warm-up here: under a counter collection every launch is slow)
        ms = time_loop(w.step, args.steps, args.warmup, warm_seconds=0.0)
        log(f"[bench] select-only {args.workload}: {ms * 1e3:.2f} us/step")
        return

    if args.lmhead_only:
        import dflash2_draft_candidate_amd as d2
        ls = synth.LM_CONFIGS["lmhead-qwen3-8b-b1"]
        hb, wb = synth.lmhead_inputs(ls.R, ls.H, ls.V, ls.seed)
        h, wt = synth.as_torch(hb, device), synth.as_torch(wb, device)
        del hb, wb
        ms = time_loop(lambda i: d2.lmhead_topk(h, wt, ls.k), args.steps, args.warmup,
                       warm_seconds=0.0)
        log(f"[bench] lmhead-only {ls.name}: {ms * 1e3:.2f} us/call, "
            f"{2 * ls.V * ls.H / (ms * 1e-3) / 1e9:.1f} GB/s of weight")
        return

    if args.k1_only:
        w = Workload(args.workload, device)
        s = w.s
        ids = torch.empty((s.R, s.k), dtype=torch.int32, device=device)
        unary = torch.empty((s.R, s.k), dtype=torch.float32, device=device)
        lse = torch.empty((s.R,), dtype=torch.float32, device=device)
        import dflash2_draft_candidate_amd as d2
        wsb = d2.library().dflash2_topk_lse_workspace_bytes(
            s.R, s.V, s.k, d2.BF16 if s.logits_dtype == "bf16" else d2.F32)
        ws = torch.empty(max(16, wsb), dtype=torch.uint8, device=device)
        # (no time-based warm-up here: under a counter collection every launch is slow)
        ms = time_loop(lambda i: w.k1_step(i, ids, unary, lse, ws), args.steps, args.warmup,
                       warm_seconds=0.0)
        log(f"[bench] k1-only {args.workload}: {ms * 1e3:.2f} us/launch, "
            f"{k1_bytes(s) / (ms * 1e-3) / 1e9:.1f} GB/s")
        if args.copy_mib > 0:
            n = args.copy_mib << 20
            src = torch.empty(n, dtype=torch.uint8, device=device).fill_(1)
            dst = torch.empty_like(src)
            for _ in range(COPY_REPS):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"[bench] {COPY_REPS} device copies of {args.copy_mib} MiB done")
        return

    main_res = measure(args.workload, device, args.steps, args.warmup)
    main_w = main_res.pop("_workload")
    s = main_w.s
    extras = {"walk_modes": measure_modes(main_w, args.steps, args.warmup),
              "gate": measure_gate(main_w, args.steps, args.warmup),
              "dynconv": measure_dynconv(device, args.steps, args.warmup),
              "lmhead_topk": measure_lmhead(device, args.steps, args.warmup)}
    log(f"[bench] extras: {extras}")
    del main_w
    log(f"[bench] {args.workload}: {main_res}")
    per_config = {args.workload: main_res}
    if not args.no_per_config:
        for name in synth.CONFIG_ORDER:
            if name == args.workload:
                continue
            r = measure(name, device, args.steps, args.warmup)
            r.pop("_workload")
            torch.cuda.empty_cache()
            per_config[name] = r
            log(f"[bench] {name}: {r}")

    traffic = committed_traffic()
    # the kernel's launch time: HIP events around graph replays of K1 launches (the eager loop's
    # per-launch time also holds the dispatch gap between launches; both are in per_config)
    g = main_res["graph"]
    roof = {"bound": "hbm", "achieved": g["k1_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": g["k1_frac"],
            "traffic": traffic["bytes_per_launch"] if traffic and
            traffic.get("workload") == args.workload else None,
            "kernel": "topk_lse_kernel", "algorithmic_bytes_per_launch": k1_bytes(s),
            "launch_us": g["k1_us"], "timing": "graph replay of K1 launches, HIP events",
            "eager_launch_us": main_res["k1_us"]}
    line = {
        "metric": METRIC,
        "value": main_res["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warm_seconds": WARM_SECONDS,
        "ms_per_step": round(main_res["e2e_us"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": s.B, "L": s.L, "k": s.k, "V": s.V, "H": s.H,
                   "r": s.r, "logits_dtype": s.logits_dtype, "act_dtype": s.act_dtype,
                   "codebook_dtype": s.cb_dtype, "global_batch": s.B, "seq_len": s.L,
                   "parallelism": "single-gpu"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    line["per_config"] = per_config
    line["extras"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
