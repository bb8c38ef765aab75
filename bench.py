"""Benchmark of the ternary-weight linear layer on one MI355X.

One step = one decode pass (T = 1) through the two 27B-class layer shapes,
gate/up (K=5120 -> N=34816) and down (K=17408 -> N=5120), with weights
rotated over enough device copies (> 512 MB) that every step streams them
from HBM rather than from the 256 MiB Infinity Cache. The headline value is
the whole step's algorithmic bytes per second (GB/s = 1e9 B/s). The same
line reports the s8 prefill rung at T = 2048 on the same two shapes in int8
TOPS, the draft-verify batches T = 2..16 in GB/s, the 64-layer stack, the
roofline fraction of the dominant kernel of each, and the CPU oracle timed
on the host as a baseline.

Timing: the K timed steps are captured once into a HIP graph (PyTorch's
CUDAGraph on ROCm) and replayed between HIP events recorded on the same
stream, so host launch overhead does not enter the measurement. The spread
(p10 / p50 / p90 per step) comes from 20 replays of a graph of K / 20 steps,
each between its own events. Each T <= 16 launch is also rated against the
self-measured streaming-read ceiling: the fastest of a few plans of a
read-only kernel (tern_stream_read) over the same number of bytes, from
buffers rotated past the Infinity Cache like the weights.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8.0 TB/s
I8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, 5.0 POPS
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
MALL_BYTES = 256 * 2**20
ROTATE_BYTES = 600e6  # > 2x the Infinity Cache
METRIC = "ternary linear HBM GB/s (% peak) at T=1; int8 TOPS (% peak) at T=2048"
# Sources of the kernels whose HBM traffic is stored (gemv, quant, s8, bf16
# prefill, activation-tiled small-T) and of
# their launch plans: a change to any of them voids the stored counters.
KERNEL_SRCS = [os.path.join(ROOT, "ternary_weight_linear_amd", "csrc", f)
               for f in ("tern_limb.hip", "tern_s8.hip", "tern_s8mma.hip", "tern_b16mma.hip",
                         "tern_tile.hip", "tern_limbtile.hip", "tern_chain.hip", "tern_narrow.hip", "tern_device.h",
                         "tern_internal.h", "tern_host.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(T, n, k, group):
    """Codes (2 bits/weight) + fp16 scales + bf16 activations + fp32 outputs."""
    return n * k // 4 + 2 * n * (k // group) + 2 * T * k + 4 * T * n


def kernel_source_sha():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha") != kernel_source_sha():
        return None
    v = d.get("kernels", {}).get(kernel_key)
    return None if v is None else v.get("bytes_per_launch")


def graph_time(torch, fn, steps, warmup):
    """Capture `steps` calls of fn(i) into one graph; return seconds per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(1, warmup)):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()  # untimed warm replay
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    g.replay()
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3


def event_time(torch, fn, reps, warmup=2):
    """Seconds per call of fn() (one launch each), timed between events on
    the current stream over `reps` calls after `warmup` untimed ones."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) * 1e-3 / reps


def dec_bytes_of(layers):
    return sum(algorithmic_bytes(1, b.n, b.k, b.group) for L in layers for b in L)


def graph_batches(torch, fn, warmup, per=50, batches=20):
    """The spread of per-step times: a graph of `per` steps captured once and
    replayed `batches` times, each replay between its own events (so each
    batch also carries one graph launch, about 1-2 us over `per` steps).
    Returns (mean, p10, p50, p90) seconds per step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(max(1, warmup)):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(per):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e-3 / per for a, b in ev])
    return (float(t.mean()),) + tuple(float(v) for v in np.percentile(t, [10, 50, 90]))


def read_ceiling(torch, tl, dev, nbytes, reps=100):
    """Self-measured streaming-read ceiling for one launch over `nbytes`: the
    fastest of a few (depth, waves per CU) plans of the read-only kernel,
    rotating over a pool larger than the Infinity Cache. Returns seconds per
    launch."""
    nb = (nbytes + 1023) // 1024 * 1024
    pool_bytes = max(int(ROTATE_BYTES) + nb, 2 * nb) // 4096 * 4096 + 4096
    pool = torch.ones((pool_bytes,), dtype=torch.uint8, device=dev)
    sink = torch.zeros((1,), dtype=torch.int32, device=dev)
    nslots = max(2, (pool_bytes - nb) // ((nb + 4095) // 4096 * 4096))
    stride = (pool_bytes - nb) // nslots // 4096 * 4096
    best = None
    for depth in (4, 8, 16):
        for waves in (4, 8, 16):
            def one(i, depth=depth, waves=waves):
                off = (i % nslots) * stride
                tl.stream_read(pool[off:off + nb], depth=depth, waves_per_cu=waves, sink=sink)
            t = graph_time(torch, one, reps, 3) / reps
            if best is None or t < best[0]:
                best = (t, depth, waves)
    del pool
    torch.cuda.empty_cache()
    return best


def _host_cpu():
    """(threads to use, nproc, CPU model) of the host the bench runs on."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(avail, int(cap)) if cap.isdigit() and int(cap) > 0 else avail
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, os.cpu_count() or 1, model


def _row_blocks(n, parts):
    edges = np.linspace(0, n, parts + 1).astype(int)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def cpu_baseline(ts, wts_list, x_list, budget_s=8.0):
    """The CPU oracle as it stands (plain C, one call per row block), on all
    the host's cores: a thread pool over disjoint row blocks of each matrix
    (ctypes releases the GIL during each oracle call; oracle.c itself stays
    single-threaded). The headline figure is the T=1 decode step (gate_up +
    down) in GB/s; per_config adds the small case, a draft-verify batch and
    the s8 prefill at T=2048 (codes and scales of the whole batch, the
    contraction on a sample of output rows, extrapolated to all rows and
    labelled so)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    threads, nproc, model = _host_cpu()
    pool = ThreadPoolExecutor(threads)

    def bf16_full(x, w, s):
        blocks = _row_blocks(w.shape[0], 4 * threads)
        list(pool.map(lambda r: oracle.linear_bf16(x, w[r[0]:r[1]], s[r[0]:r[1]]), blocks))

    # config 2: the decode step, as many full steps as fit the budget
    step_bytes = sum(algorithmic_bytes(1, w.shape.n, w.shape.k, w.shape.group) for w in wts_list)
    reps, t0 = 0, time.perf_counter()
    while True:
        for w, x in zip(wts_list, x_list):
            bf16_full(x, w.w, w.s)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    per_config = {"decode_T1": {"GB/s": round(reps * step_bytes / el / 1e9, 4),
                                "us_per_step": round(el / reps * 1e6, 1),
                                "sample": f"{reps} full decode steps"}}
    # config 1: the small case, T = 1 and 4
    sw = ts.weights(ts.SMALL)
    for T in (1, 4):
        xs = ts.activations(sw, T)
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 0.3:
            oracle.linear_bf16(xs, sw.w, sw.s)
            n += 1
        per_config[f"small_T{T}"] = {"us_per_call": round((time.perf_counter() - t0) / n * 1e6, 2)}
    # config 3: a draft-verify batch (T = 8) through gate_up and down, in full
    T = 8
    xs8 = [ts.activations(w, T) for w in wts_list]
    t0 = time.perf_counter()
    for w, x in zip(wts_list, xs8):
        bf16_full(x, w.w, w.s)
    el = time.perf_counter() - t0
    b8 = sum(algorithmic_bytes(T, w.shape.n, w.shape.k, w.shape.group) for w in wts_list)
    per_config["draft_verify_T8"] = {"GB/s": round(b8 / el / 1e9, 4), "ms": round(el * 1e3, 1)}
    # config 4: s8 at T = 2048 on gate_up; quantisation of the whole batch,
    # contraction on sampled output rows, extrapolated to every row
    w = wts_list[0]
    T, rows = 2048, 256
    xq = ts.activations(w, T)
    t0 = time.perf_counter()
    tb = _row_blocks(T, threads)
    qs = list(pool.map(lambda r: oracle.quant_s8(xq[r[0]:r[1]]), tb))
    tq = time.perf_counter() - t0
    q = np.concatenate([a for a, _ in qs])
    sc = np.concatenate([b for _, b in qs])
    pick = np.random.default_rng(4).choice(w.shape.n, rows, replace=False)
    ws_, ss_ = w.w[pick], w.s[pick]
    t0 = time.perf_counter()
    list(pool.map(lambda r: oracle.linear_s8(q[r[0]:r[1]], sc[r[0]:r[1]], ws_, ss_), tb))
    tr = time.perf_counter() - t0
    t_full = tq + tr * w.shape.n / rows
    ops = 2 * T * w.shape.n * w.shape.k
    per_config["s8_T2048_gate_up"] = {
        "TOPS": round(ops / t_full / 1e12, 6), "s_extrapolated": round(t_full, 1),
        "sample": f"quant of all {T} tokens ({tq:.2f} s) + contraction of {rows} of {w.shape.n} rows "
                  f"({tr:.2f} s), extrapolated to every row"}
    pool.shutdown()
    return {"value": per_config["decode_T1"]["GB/s"], "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps} full T=1 decode steps (gate_up 5120->34816 + down 17408->5120) through "
                      f"oracle_linear_bf16 (fp64), {threads} threads over row blocks",
            "nproc": nproc, "cpu_model": model, "per_config": per_config}


def stack_leg(torch, ts, tl, dev, decode_reps=10, prefill_reps=2):
    """The 64-layer stack (q, k, v, o 5120->5120; gate, up 5120->17408; down
    17408->5120 per layer): one T=1 decode pass (448 calls) and one
    2048-token prefill in two 1024-token chunks (896 s8 calls), each pass
    captured in one graph and timed over several replays. Every layer has its
    own device copy of the weights (6.3 GB resident, streamed from HBM each
    pass); the copies are layer 0's matrices, drawn with layer 0's seeds."""
    base, xs1, xsp = [], [], []
    for proj in range(len(ts.STACK_PROJ)):
        w = ts.weights(ts.stack_shape(0, proj))
        base.append(tl.TernaryWeights.from_host(w.w, w.s, device=dev))
        xs1.append(torch.from_numpy(ts.activations(w, 1).view(np.int16)).to(dev).view(torch.bfloat16))
        xsp.append(torch.from_numpy(ts.activations(w, 2048).view(np.int16)).to(dev).view(torch.bfloat16))
    layers = [base] + [[tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group)
                        for b in base] for _ in range(ts.STACK_LAYERS - 1)]
    nbytes = sum(b.nbytes for L in layers for b in L)
    y1 = [torch.empty((1, b.n), dtype=torch.float32, device=dev) for b in base]
    yp = [torch.empty((1024, b.n), dtype=torch.float32, device=dev) for b in base]
    wsz = max(tl.workspace_bytes(1024, b.n, b.k, b.group) for b in base)
    wsp = torch.zeros((wsz,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    log(f"stack: {ts.STACK_LAYERS} layers x {len(base)} projections, {nbytes / 1e9:.2f} GB resident")

    def decode_pass(_):
        for L in layers:
            for j, b in enumerate(L):
                tl.linear(xs1[j], b, y=y1[j])

    def prefill_pass(_):
        for c in range(2):
            for L in layers:
                for j, b in enumerate(L):
                    tl.linear(xsp[j][1024 * c:1024 * (c + 1)], b, y=yp[j], workspace=wsp)

    t_dec = graph_time(torch, decode_pass, decode_reps, 1) / decode_reps
    ops = sum(2 * 2048 * b.n * b.k for L in layers for b in L)

    # The same decode pass as one persistent launch (tern_linear_chain). As
    # the stack is defined here every projection reads its own synthetic x, so
    # the chain needs no waits; a second chain adds the waits a layer would
    # have if outputs were chained (q, k, v after the previous layer's down,
    # o after v, gate and up after o, down after up): each is a device-wide
    # drain.
    def chain_items(Ls, xs, ys, deps):
        items = []
        for L in Ls:
            base = len(items)
            for j, b in enumerate(L):
                d = deps[j]
                after = -1 if d is None else (base + d if d >= 0 else (base - 1 if base > 0 else -1))
                items.append((b, xs[j], ys[j], None, after))
        return items

    # offsets within a layer (-1: the previous layer's last item; None: no wait)
    ch = tl.Chain(chain_items(layers, xs1, y1, [None] * 7), device=dev)
    t_chain = event_time(torch, ch.run, decode_reps)
    assert not ch.failed()
    del ch
    ch = tl.Chain(chain_items(layers, xs1, y1, [-1, -1, -1, 2, 3, 3, 5]), device=dev)
    t_chain_w = event_time(torch, ch.run, decode_reps)
    assert not ch.failed()
    del ch
    log(f"stack decode pass as one chain launch: {t_chain * 1e3:.3f} ms ({dec_bytes_of(layers) / t_chain / 1e9:.0f} GB/s); "
        f"with the layer's 4 waits: {t_chain_w * 1e3:.3f} ms ({dec_bytes_of(layers) / t_chain_w / 1e9:.0f} GB/s)")
    t_pre = graph_time(torch, prefill_pass, prefill_reps, 1) / prefill_reps
    dec_bytes = sum(algorithmic_bytes(1, b.n, b.k, b.group) for L in layers for b in L)
    log(f"stack decode pass {t_dec * 1e3:.3f} ms ({dec_bytes / t_dec / 1e9:.0f} GB/s), "
        f"prefill pass {t_pre * 1e3:.2f} ms ({ops / t_pre / 1e12:.0f} TOPS)")

    # Fused variant: q|k|v and gate|up share their input, so each pair or
    # triple is one matrix (the packed layout is strip-major, so stacking
    # along N is concatenating the code and scale buffers): 4 launches per
    # layer instead of 7, the same bytes.
    del layers
    torch.cuda.empty_cache()
    groups = [(0, 1, 2), (3,), (4, 5), (6,)]

    def fuse(parts):
        if len(parts) == 1:
            b = base[parts[0]]
            return tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group)
        bs = [base[i] for i in parts]
        return tl.TernaryWeights(torch.cat([b.codes for b in bs]), torch.cat([b.scales for b in bs]),
                                 sum(b.n for b in bs), bs[0].k, bs[0].group)

    flayers = [[fuse(g) for g in groups] for _ in range(ts.STACK_LAYERS)]
    fx1 = [xs1[g[0]] for g in groups]
    fxp = [xsp[g[0]] for g in groups]
    fy1 = [torch.empty((1, b.n), dtype=torch.float32, device=dev) for b in flayers[0]]
    fyp = [torch.empty((1024, b.n), dtype=torch.float32, device=dev) for b in flayers[0]]
    fwsz = max(tl.workspace_bytes(1024, b.n, b.k, b.group) for b in flayers[0])
    fwsp = torch.zeros((fwsz,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def fdecode_pass(_):
        for L in flayers:
            for j, b in enumerate(L):
                tl.linear(fx1[j], b, y=fy1[j])

    def fprefill_pass(_):
        for c in range(2):
            for L in flayers:
                for j, b in enumerate(L):
                    tl.linear(fxp[j][1024 * c:1024 * (c + 1)], b, y=fyp[j], workspace=fwsp)

    f_dec = graph_time(torch, fdecode_pass, decode_reps, 1) / decode_reps
    fch = tl.Chain(chain_items(flayers, fx1, fy1, [None] * 4), device=dev)
    f_chain = event_time(torch, fch.run, decode_reps)
    assert not fch.failed()
    del fch
    f_pre = graph_time(torch, fprefill_pass, prefill_reps, 1) / prefill_reps
    f_bytes = sum(algorithmic_bytes(1, b.n, b.k, b.group) for L in flayers for b in L)
    log(f"stack, fused q|k|v and gate|up: decode pass {f_dec * 1e3:.3f} ms "
        f"({f_bytes / f_dec / 1e9:.0f} GB/s; one chain launch {f_chain * 1e3:.3f} ms, "
        f"{f_bytes / f_chain / 1e9:.0f} GB/s), prefill pass {f_pre * 1e3:.2f} ms ({ops / f_pre / 1e12:.0f} TOPS)")
    return {"workload": "64-layer stack, 448 projections (6.33 GB packed); decode T=1 pass; "
                        "2048-token prefill in two 1024-token chunks (s8)",
            "decode": {"ms_per_pass": round(t_dec * 1e3, 4), "GB/s": round(dec_bytes / t_dec / 1e9, 1),
                       "frac_of_hbm_peak": round(dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS, 4),
                       "launches": ts.STACK_LAYERS * len(base)},
            "decode_chain": {"ms_per_pass": round(t_chain * 1e3, 4), "GB/s": round(dec_bytes / t_chain / 1e9, 1),
                             "frac_of_hbm_peak": round(dec_bytes / t_chain / 1e9 / HBM_PEAK_GBS, 4),
                             "launches": 1,
                             "kernel": "tern_chain_kernel: the 448 projections in one persistent launch"},
            "decode_chain_with_layer_waits": {
                "ms_per_pass": round(t_chain_w * 1e3, 4), "GB/s": round(dec_bytes / t_chain_w / 1e9, 1),
                "waits": 4 * ts.STACK_LAYERS,
                "note": "q, k, v after the previous layer's down; o after v; gate, up after o; down after up"},
            "prefill": {"ms_per_pass": round(t_pre * 1e3, 3), "TOPS": round(ops / t_pre / 1e12, 1),
                        "frac_of_i8_peak": round(ops / t_pre / 1e12 / I8_PEAK_TOPS, 4),
                        "tokens_per_s": round(2048 / t_pre, 1)},
            "fused_qkv_gate_up": {
                "launches_per_pass": ts.STACK_LAYERS * len(groups),
                "decode": {"ms_per_pass": round(f_dec * 1e3, 4), "GB/s": round(f_bytes / f_dec / 1e9, 1),
                           "frac_of_hbm_peak": round(f_bytes / f_dec / 1e9 / HBM_PEAK_GBS, 4)},
                "decode_chain": {"ms_per_pass": round(f_chain * 1e3, 4), "GB/s": round(f_bytes / f_chain / 1e9, 1),
                                 "frac_of_hbm_peak": round(f_bytes / f_chain / 1e9 / HBM_PEAK_GBS, 4),
                                 "launches": 1},
                "prefill": {"ms_per_pass": round(f_pre * 1e3, 3), "TOPS": round(ops / f_pre / 1e12, 1),
                            "tokens_per_s": round(2048 / f_pre, 1)}}}


def t5_bytes(T, n, k, group):
    """Base-3 codes (13 bytes per 64 weights) + fp16 scales + bf16 x + fp32 y."""
    return n * (k // 1024) * 208 + 2 * n * (k // group) + 2 * T * k + 4 * T * n


def t5_leg(torch, ts, tl, dev, wts, steps=200, rounds=3):
    """A/B of the T=1 gemv on the same matrices packed 2-bit (v1) and base-3
    (t5, five weights per byte): the arms alternate `rounds` times, each a
    graph of `steps` launches over weight copies rotated past the Infinity
    Cache; per arm the median of the rounds."""
    out = {}
    for w in wts:
        shape = w.shape
        x = torch.from_numpy(ts.activations(w, 1).view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((1, shape.n), dtype=torch.float32, device=dev)
        arms = {}
        for layout in ("v1", "t5"):
            b = tl.TernaryWeights.from_host(w.w, w.s, device=dev, layout=layout)
            nsets = max(2, math.ceil(ROTATE_BYTES / b.nbytes))
            arms[layout] = [b] + [tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group,
                                                    layout) for _ in range(nsets - 1)]
        times = {"v1": [], "t5": []}
        for _ in range(rounds):
            for layout in ("v1", "t5"):
                sets = arms[layout]

                def one(i, sets=sets):
                    tl.linear(x, sets[i % len(sets)], y=y)
                times[layout].append(graph_time(torch, one, steps, 10) / steps)
        e = {}
        for layout, fb in (("v1", algorithmic_bytes), ("t5", t5_bytes)):
            t = float(np.median(times[layout]))
            by = fb(1, shape.n, shape.k, shape.group)
            e[layout] = {"us": round(t * 1e6, 3), "bytes": by, "GB/s": round(by / t / 1e9, 1),
                         "us_rounds": [round(v * 1e6, 3) for v in times[layout]]}
        e["t5_speedup"] = round(e["v1"]["us"] / e["t5"]["us"], 4)
        out[shape.name] = e
        log(f"  t5 A/B {shape.name}: v1 {e['v1']['us']:.2f} us, t5 {e['t5']['us']:.2f} us "
            f"({e['t5_speedup']:.3f}x; t5 bytes {e['t5']['bytes'] / 1e6:.2f} MB)")
        del arms
        torch.cuda.empty_cache()
    return {"workload": "gemv T=1 on gate_up and down, the same weights packed 2-bit (v1) and "
                        "base-3 (t5: 5 weights per byte + fp16 scale per 128)", "per_shape": out}


SMALL_T = (2, 4, 8, 12, 16)


def small_t_leg(torch, ts, tl, dev, steps=1000):
    """The draft-verify batches: T in {2, 4, 8, 12, 16} through gate_up, down
    and the 5120 -> 5120 out-projection with the rung the dispatcher picks
    (small_t for T <= 8, small_t_tiled above), weights rotated over > 600 MB
    so that they stream from HBM. Algorithmic bytes per launch as for T = 1
    (codes + scales + x + y); GB/s is that over the mean event-timed launch
    of 20 replays of a 50-launch graph (the spread over the replays is kept
    as p10 / p50 / p90)."""
    out = {}
    for shape in (ts.GATE_UP, ts.DOWN, ts.OUT_PROJ):
        w = ts.weights(shape)
        base = tl.TernaryWeights.from_host(w.w, w.s, device=dev)
        nsets = max(2, math.ceil(ROTATE_BYTES / base.nbytes))
        sets = [base] + [tl.TernaryWeights(base.codes.clone(), base.scales.clone(), base.n, base.k,
                                           base.group) for _ in range(nsets - 1)]
        per_t = {}
        for T in SMALL_T:
            x = torch.from_numpy(ts.activations(w, T).view(np.int16)).to(dev).view(torch.bfloat16)
            y = torch.empty((T, shape.n), dtype=torch.float32, device=dev)
            wsz = tl.workspace_bytes(T, shape.n, shape.k, shape.group)
            wsp = torch.zeros((max(1, wsz),), dtype=torch.uint8, device=dev)
            rung = tl.resolve_rung(T)

            def one(i):
                tl.linear(x, sets[i % nsets], y=y, workspace=wsp)

            t, p10, p50, p90 = graph_batches(torch, one, 5, per=steps // 20)
            b = algorithmic_bytes(T, shape.n, shape.k, shape.group)
            per_t[f"T{T}"] = {"rung": rung, "us_per_launch": round(t * 1e6, 2),
                              "us_p10_p50_p90": [round(v * 1e6, 2) for v in (p10, p50, p90)],
                              "GB/s": round(b / t / 1e9, 1),
                              "frac_of_hbm_peak": round(b / t / 1e9 / HBM_PEAK_GBS, 4)}
            log(f"  small-T {shape.name} T={T} ({rung}): {t * 1e6:.2f} us (p10/p50/p90 {p10 * 1e6:.2f}/"
                f"{p50 * 1e6:.2f}/{p90 * 1e6:.2f}), {b / t / 1e9:.0f} GB/s")
        # the read ceiling for each launch's bytes, after the layer's timings
        for T in SMALL_T:
            e = per_t[f"T{T}"]
            tc = read_ceiling(torch, tl, dev, algorithmic_bytes(T, shape.n, shape.k, shape.group), reps=50)[0]
            e["read_ceiling_us"] = round(tc * 1e6, 2)
            e["frac_of_read_ceiling"] = round(tc * 1e6 / e["us_per_launch"], 4)
        log(f"  small-T {shape.name}: read ceiling " + ", ".join(
            f"T={T} {per_t[f'T{T}']['read_ceiling_us']:.2f} us ({per_t[f'T{T}']['frac_of_read_ceiling']:.0%})"
            for T in SMALL_T))
        out[shape.name] = per_t
        del sets, base
        torch.cuda.empty_cache()
    return {"workload": "draft-verify batches T in {2,4,8,12,16} on gate_up 5120->34816, "
                        "down 17408->5120 and o_proj 5120->5120", "per_shape": out}


def kernels_only(torch, ts, tl, dev, n):
    """For rocprofv3 --pmc runs, all on gate_up with weights rotated over
    > 512 MB: n launches of the gemv kernel (T=1), n/10 of the s8 rung (quant
    + contraction, T=2048), n/10 of the bf16 prefill (T=2048), n of the T=8
    draft-verify batch, n of the rotated quantisation (T=2048), n of the gemv
    on base-3 (t5) weights, n of the decode step (gate_up + down) as one
    chain launch, n each of down and o_proj at T = 1, 4 and 16, then plain
    64 MiB device copies whose byte counters calibrate FETCH_SIZE /
    WRITE_SIZE."""
    w = ts.weights(ts.GATE_UP)
    b = tl.TernaryWeights.from_host(w.w, w.s, device=dev)
    sets = [b] + [tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group)
                  for _ in range(max(1, math.ceil(ROTATE_BYTES / b.nbytes)) - 1)]
    x1 = torch.from_numpy(ts.activations(w, 1).view(np.int16)).to(dev).view(torch.bfloat16)
    y1 = torch.empty((1, b.n), dtype=torch.float32, device=dev)
    T = 2048
    x8 = torch.from_numpy(ts.activations(w, T).view(np.int16)).to(dev).view(torch.bfloat16)
    y8 = torch.empty((T, b.n), dtype=torch.float32, device=dev)
    ws = torch.zeros((tl.workspace_bytes(T, b.n, b.k, b.group),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for i in range(n):
        tl.linear(x1, sets[i % len(sets)], y=y1)
    torch.cuda.synchronize()
    for i in range(max(1, n // 10)):
        tl.linear(x8, sets[i % len(sets)], y=y8, workspace=ws)
    torch.cuda.synchronize()
    for i in range(max(1, n // 10)):  # bf16 prefill (small_t_tiled above 16 tokens)
        tl.linear(x8, sets[i % len(sets)], rung="small_t_tiled", y=y8)
    torch.cuda.synchronize()
    x16 = torch.from_numpy(ts.activations(w, 8).view(np.int16)).to(dev).view(torch.bfloat16)
    y16 = torch.empty((8, b.n), dtype=torch.float32, device=dev)
    for i in range(n):  # draft-verify batch T = 8 (resident limb kernel on this wide layer)
        tl.linear(x16, sets[i % len(sets)], y=y16)
    torch.cuda.synchronize()
    qr = torch.empty((T, b.k), dtype=torch.int8, device=dev)
    sr = torch.empty((T,), dtype=torch.float32, device=dev)
    for i in range(n):  # rotated quantisation of the T = 2048 prefill activations
        tl.quant_act_s8_rot(x8, q=qr, scale=sr, layout="operand_order")
    torch.cuda.synchronize()
    del sets
    torch.cuda.empty_cache()
    b5 = tl.TernaryWeights.from_host(w.w, w.s, device=dev, layout="t5")
    s5 = [b5] + [tl.TernaryWeights(b5.codes.clone(), b5.scales.clone(), b5.n, b5.k, b5.group, "t5")
                 for _ in range(max(1, math.ceil(ROTATE_BYTES / b5.nbytes)) - 1)]
    for i in range(n):  # gemv on base-3 (t5) weights
        tl.linear(x1, s5[i % len(s5)], y=y1)
    torch.cuda.synchronize()
    del s5, b5
    wd = ts.weights(ts.DOWN)
    bd = tl.TernaryWeights.from_host(wd.w, wd.s, device=dev)
    xd = torch.from_numpy(ts.activations(wd, 1).view(np.int16)).to(dev).view(torch.bfloat16)
    yd = torch.empty((1, bd.n), dtype=torch.float32, device=dev)
    nch = max(2, math.ceil(ROTATE_BYTES / (b.nbytes + bd.nbytes)))
    chains = []
    for _ in range(nch):
        bg = tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group)
        bdd = tl.TernaryWeights(bd.codes.clone(), bd.scales.clone(), bd.n, bd.k, bd.group)
        chains.append(tl.Chain([(bg, x1, y1, None, -1), (bdd, xd, yd, None, -1)], device=dev))
    for i in range(n):  # the decode step (gate_up + down) as one chain launch
        chains[i % nch].run()
    torch.cuda.synchronize()
    del chains
    # narrow layers (down 17408 -> 5120, o_proj 5120 -> 5120): the gemv (T = 1)
    # and the draft-verify kernels at T = 4 and T = 16, weights rotated likewise
    for shape in (ts.DOWN, ts.OUT_PROJ):
        wn = ts.weights(shape)
        bn = tl.TernaryWeights.from_host(wn.w, wn.s, device=dev)
        sn = [bn] + [tl.TernaryWeights(bn.codes.clone(), bn.scales.clone(), bn.n, bn.k, bn.group)
                     for _ in range(max(1, math.ceil(ROTATE_BYTES / bn.nbytes)) - 1)]
        for T in (1, 4, 16):
            xn = torch.from_numpy(ts.activations(wn, T).view(np.int16)).to(dev).view(torch.bfloat16)
            yn = torch.empty((T, bn.n), dtype=torch.float32, device=dev)
            wsn = torch.zeros((max(1, tl.workspace_bytes(T, bn.n, bn.k, bn.group)),), dtype=torch.uint8, device=dev)
            for i in range(n):
                tl.linear(xn, sn[i % len(sn)], y=yn, workspace=wsn)
            torch.cuda.synchronize()
        del sn, bn
        torch.cuda.empty_cache()
    src = torch.empty(64 * 2**20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("kernels-only done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--s8-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-s8", action="store_true")
    ap.add_argument("--no-stack", action="store_true", help="skip the 64-layer stack passes")
    ap.add_argument("--no-small-t", action="store_true", help="skip the T = 2..16 batches")
    ap.add_argument("--no-t5", action="store_true", help="skip the 2-bit / base-3 gemv A/B")
    ap.add_argument("--kernels-only", action="store_true",
                    help="plain launches of the two dominant kernels and a 64 MiB copy, for "
                         "rocprofv3 counter runs (no timing, no JSON line)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the layer is not sharded across "
              "GPUs); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import tern_synth as ts
    import ternary_weight_linear_amd as tl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tl.lib()

    if args.kernels_only:
        kernels_only(torch, ts, tl, dev, args.steps)
        return

    shapes = (ts.GATE_UP, ts.DOWN)
    log("drawing weights")
    wts = [ts.weights(s) for s in shapes]
    base = [tl.TernaryWeights.from_host(w.w, w.s, device=dev) for w in wts]
    step_bytes = sum(algorithmic_bytes(1, s.n, s.k, s.group) for s in shapes)
    nsets = max(2, math.ceil(ROTATE_BYTES / step_bytes))
    sets = [base]
    for _ in range(nsets - 1):
        sets.append([tl.TernaryWeights(b.codes.clone(), b.scales.clone(), b.n, b.k, b.group)
                     for b in base])
    torch.cuda.synchronize()
    log(f"{nsets} rotation sets x {step_bytes / 1e6:.2f} MB")

    xb = [ts.activations(w, 1) for w in wts]
    x1 = [torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16) for b in xb]
    y1 = [torch.empty((1, s.n), dtype=torch.float32, device=dev) for s in shapes]
    assert tl.resolve_rung(1) == "gemv"

    def decode_step(i):
        ws = sets[i % nsets]
        tl.linear(x1[0], ws[0], y=y1[0])
        tl.linear(x1[1], ws[1], y=y1[1])

    K, Wm = args.steps, args.warmup
    el = graph_time(torch, decode_step, K, Wm)
    value = K * step_bytes / el / 1e9
    ms_per_step = el / K * 1e3
    _, d10, d50, d90 = graph_batches(torch, decode_step, Wm)
    log(f"decode step {ms_per_step * 1e3:.2f} us, {value:.1f} GB/s (per-step p10/p50/p90 "
        f"{d10 * 1e6:.2f}/{d50 * 1e6:.2f}/{d90 * 1e6:.2f} us over 20 batches of 50)")

    per_shape = {}
    for j, s in enumerate(shapes):
        def one(i, j=j):
            tl.linear(x1[j], sets[i % nsets][j], y=y1[j])
        t = graph_time(torch, one, K, Wm) / K
        _, p10, p50, p90 = graph_batches(torch, one, Wm)
        b = algorithmic_bytes(1, s.n, s.k, s.group)
        per_shape[s.name] = {"rung": "gemv", "us_per_launch": round(t * 1e6, 3),
                             "us_p10_p50_p90": [round(v * 1e6, 3) for v in (p10, p50, p90)],
                             "bytes": b, "GB/s": round(b / t / 1e9, 1)}
        log(f"  {s.name}: {t * 1e6:.2f} us/launch (p10/p50/p90 {p10 * 1e6:.2f}/{p50 * 1e6:.2f}/"
            f"{p90 * 1e6:.2f}), {b / t / 1e9:.1f} GB/s")
    for s in shapes:  # the read ceiling for the same bytes, after the layer timings
        e = per_shape[s.name]
        tc, dc, wc = read_ceiling(torch, tl, dev, e["bytes"])
        e["read_ceiling"] = {"us": round(tc * 1e6, 3), "GB/s": round(e["bytes"] / tc / 1e9, 1),
                             "depth": dc, "waves_per_cu": wc}
        e["frac_of_read_ceiling"] = round(tc * 1e6 / e["us_per_launch"], 4)
        log(f"  {s.name}: read ceiling {tc * 1e6:.2f} us ({e['bytes'] / tc / 1e9:.0f} GB/s); the "
            f"kernel reaches {e['frac_of_read_ceiling']:.0%} of it")
    # Context: the same step as one persistent launch (tern_linear_chain, the
    # two projections with their own inputs, no wait between them) over the
    # same rotated weight sets.
    chains = [tl.Chain([(sets[i][0], x1[0], y1[0], None, -1), (sets[i][1], x1[1], y1[1], None, -1)], device=dev)
              for i in range(nsets)]
    t_ch = event_time(torch, lambda: [c.run() for c in chains], max(1, K // nsets)) / nsets
    assert not any(c.failed() for c in chains)
    del chains
    log(f"decode step as one chain launch: {t_ch * 1e6:.2f} us ({step_bytes / t_ch / 1e9:.1f} GB/s)")

    dom = shapes[0].name
    achieved = per_shape[dom]["GB/s"]
    traffic = stored_traffic(f"gemv:{dom}")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": f"tern_limb_kernel (gemv rung, T=1) on {dom}",
                "algorithmic_bytes_per_launch": per_shape[dom]["bytes"],
                "us_per_launch": per_shape[dom]["us_per_launch"],
                "read_ceiling_GB/s": per_shape[dom]["read_ceiling"]["GB/s"],
                "frac_of_read_ceiling": per_shape[dom]["frac_of_read_ceiling"]}
    ceil_step = sum(v["read_ceiling"]["us"] for v in per_shape.values()) * 1e-6

    s8 = None
    if not args.no_s8:
        T = 2048
        xs = [torch.from_numpy(ts.activations(w, T).view(np.int16)).to(dev).view(torch.bfloat16)
              for w in wts]
        ys = [torch.empty((T, s.n), dtype=torch.float32, device=dev) for s in shapes]
        wsz = max(tl.workspace_bytes(T, s.n, s.k, s.group) for s in shapes)
        wsp = torch.zeros((wsz,), dtype=torch.uint8, device=dev)
        qs = [tl.quant_act_s8(x, layout="operand_order") for x in xs]
        assert tl.resolve_rung(T) == "s8"
        ops = sum(2 * T * s.n * s.k for s in shapes)
        K8 = args.s8_steps

        def prefill_step(i):
            for j in range(2):
                tl.linear(xs[j], sets[i % nsets][j], y=ys[j], workspace=wsp)

        el8 = graph_time(torch, prefill_step, K8, 2)
        tops = K8 * ops / el8 / 1e12
        gemm = {}
        for j, s in enumerate(shapes):
            def g1(i, j=j):
                tl.linear_s8_q(qs[j][0], qs[j][1], sets[i % nsets][j], y=ys[j],
                               layout="operand_order")
            t = graph_time(torch, g1, K8, 2) / K8
            _, g10, g50, g90 = graph_batches(torch, g1, 2, per=5)
            def q1(i, j=j):
                tl.quant_act_s8(xs[j], q=qs[j][0], scale=qs[j][1], layout="operand_order")
            tq = graph_time(torch, q1, K8, 2) / K8
            o = 2 * T * s.n * s.k
            gemm[s.name] = {"us_s8_kernel": round(t * 1e6, 2), "TOPS_s8_kernel": round(o / t / 1e12, 1),
                            "us_s8_kernel_p10_p50_p90": [round(v * 1e6, 2) for v in (g10, g50, g90)],
                            "us_quant_kernel": round(tq * 1e6, 2)}
            log(f"  s8 {s.name}: gemm {t * 1e6:.1f} us ({o / t / 1e12:.0f} TOPS; p10/p50/p90 over 20 replays "
                f"of 5: {g10 * 1e6:.1f}/{g50 * 1e6:.1f}/{g90 * 1e6:.1f} us), quant {tq * 1e6:.1f} us")
        ach = gemm[dom]["TOPS_s8_kernel"]
        s8 = {"metric": "int8 TOPS at T=2048 (quant + s8 contraction, both shapes)",
              "value": round(tops, 1), "unit": "TOPS", "ms_per_step": round(el8 / K8 * 1e3, 4),
              "steps": K8, "dtype": "i8", "per_shape": gemm,
              "roofline": {"bound": "mfma", "achieved": ach, "peak": I8_PEAK_TOPS, "unit": "TOPS",
                           "frac": round(ach / I8_PEAK_TOPS, 4),
                           "traffic": stored_traffic(f"s8:{dom}"),
                           "kernel": f"tern_s8m_kernel (s8 rung contraction) on {dom}, T={T}"}}
        log(f"s8 prefill step {el8 / K8 * 1e3:.3f} ms, {tops:.1f} TOPS")

        # The bf16 prefill path (small_t_tiled at T = 2048, where T >= 17 goes
        # with the s8 rung switched off): no activation quantisation.
        b16 = {}
        for j, s in enumerate(shapes):
            def b1(i, j=j):
                tl.linear(xs[j], sets[i % nsets][j], rung="small_t_tiled", y=ys[j], workspace=wsp)
            t = graph_time(torch, b1, K8, 2) / K8
            o = 2 * T * s.n * s.k
            b16[s.name] = {"us": round(t * 1e6, 2), "TFLOPs": round(o / t / 1e12, 1)}
            log(f"  bf16 prefill {s.name}: {t * 1e6:.1f} us ({o / t / 1e12:.0f} TFLOP/s)")
        # The rotated quantisation (1024-wide Hadamard blocks fused into the
        # int8 quantisation): HBM bound, 2 B read + 1 B written per
        # activation and 4 B per token scale.
        rq = {}
        for j, s in enumerate(shapes):
            def r1(i, j=j):
                tl.quant_act_s8_rot(xs[j], q=qs[j][0], scale=qs[j][1], layout="operand_order")
            t = graph_time(torch, r1, K8, 2) / K8
            by = 3 * T * s.k + 4 * T
            rq[s.name] = {"us": round(t * 1e6, 2), "bytes": by, "GB/s": round(by / t / 1e9, 1),
                          "us_plain_quant": gemm[s.name]["us_quant_kernel"]}
            log(f"  rotated quant K={s.k}: {t * 1e6:.1f} us ({by / t / 1e9:.0f} GB/s)")
        ach_r = rq[dom]["GB/s"]
        s8["rotated_quant"] = {
            "metric": "HBM GB/s of the fused rotate (1024-wide Hadamard) and int8 quantise kernel, T=2048",
            "per_shape": rq,
            "roofline": {"bound": "hbm", "achieved": ach_r, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach_r / HBM_PEAK_GBS, 4),
                         "traffic": stored_traffic(f"quant_rot:{dom}"),
                         "kernel": f"tern_quant_rot_kernel on the {dom} activations (K={shapes[0].k}), T={T}",
                         "algorithmic_bytes_per_launch": rq[dom]["bytes"], "us_per_launch": rq[dom]["us"]}}

        ach16 = b16[dom]["TFLOPs"]
        s8["bf16_prefill"] = {
            "metric": "bf16 TFLOP/s at T=2048 (rung small_t_tiled, no activation quantisation)",
            "per_shape": b16,
            "roofline": {"bound": "mfma", "achieved": ach16, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach16 / BF16_PEAK_TFLOPS, 4),
                         "traffic": stored_traffic(f"bf16_prefill:{dom}"),
                         "kernel": f"tern_b16m_kernel (bf16 prefill) on {dom}, T={T}"}}

    t5 = None
    if not args.no_t5:
        t5 = t5_leg(torch, ts, tl, dev, wts)

    small = None
    if not args.no_small_t:
        small = small_t_leg(torch, ts, tl, dev)

    stack = None
    if not args.no_stack:
        del sets  # the rotation copies; the stack holds 6.3 GB of its own
        torch.cuda.empty_cache()
        stack = stack_leg(torch, ts, tl, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(ts, wts, xb)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['cpu_model']}); "
            + ", ".join(f"{k}: {v}" for k, v in cpu["per_config"].items()))

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
           "warmup": Wm, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "decode T=1 through gate_up 5120->34816 and down 17408->5120, "
                                  "ternary weights (2-bit packed), fp16 scale per 128, bf16 x",
                      "T": 1, "rotation_sets": nsets, "bytes_per_step": step_bytes,
                      "per_shape": per_shape, "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                      "us_per_step_p10_p50_p90": [round(v * 1e6, 3) for v in (d10, d50, d90)],
                      "read_ceiling_us_per_step": round(ceil_step * 1e6, 3),
                      "frac_of_read_ceiling": round(ceil_step / (el / K), 4),
                      "chain_launch": {"us_per_step": round(t_ch * 1e6, 3),
                                       "GB/s": round(step_bytes / t_ch / 1e9, 1),
                                       "note": "context, not the value: both projections in one "
                                               "tern_linear_chain launch with independent inputs "
                                               "(a decode whose down reads gate_up's output waits "
                                               "between them)"}},
           "roofline": roofline, "s8_prefill": s8, "t5_gemv_ab": t5, "small_t": small, "stack": stack,
           "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
