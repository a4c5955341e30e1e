"""Benchmark of the fused 4-bit skinny GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--no-cpu]

Workload (the headline): C = A * dequant(W)^T with K=8192, N=28672 (an FFN
up-projection), blocksize 64, fp32 absmax, for M = 1, 2, 4, 8 token rows.  One
step = one dispatcher-routed q4_gemm_skinny call per M.  Inputs are seeded
synthetic data resident in HBM before timing starts.  Each launch reads a
different copy of the packed weights: the copies total >= 1 GiB, four times
the 256 MB Infinity Cache, so every timed launch streams its weights from HBM.

Printed: one JSON line with the whole-job rate (algorithmic bytes / wall time
of the K timed steps issued call by call; the same steps captured into a HIP
graph and replayed are reported beside it), per-M
kernel times from back-to-back launches (a graph replay between HIP events),
the roofline of the M=1 kernel, a CPU-oracle baseline on a bounded
sample, and (unless --quick) the other decode workloads: the 4096x4096 GEMV,
the decode layer set with its fused-vs-split crossover, the bf16 skinny GEMM
and the large-vocabulary projection.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "achieved HBM GB/s and % of peak, fused 4-bit skinny GEMM at M=1/2/4/8"
PEAK_GBS = 8000.0  # MI355X HBM3E
BS = 64
MALL_BYTES = 256 << 20
ROTATE_BYTES = 1 << 30
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "fused_q4_m1_k8192_n28672.traffic.md")
FUSED_SOURCES = [os.path.join(ROOT, "bit_dequant_skinny_amd", "csrc", f)
                 for f in ("fused_mfma.hip", "device.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def q4_bytes(M, N, K, bs=BS):
    """Algorithmic bytes of one fused call: packed W, fp32 absmax, A, C, codebook."""
    return N * K // 2 + 4 * N * K // bs + 2 * M * K + 2 * M * N + 64


def bf16_bytes(M, N, K, bias):
    return 2 * N * K + 2 * M * K + 2 * M * N + (2 * N if bias else 0)


class Dev:
    def __init__(self):
        import torch
        self.t = torch
        self.dev = torch.device("cuda:0")

    def bf16(self, a):
        t = self.t
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(t.bfloat16).to(self.dev)

    def raw(self, a):
        return self.t.from_numpy(np.ascontiguousarray(a)).to(self.dev)

    def copies(self, tensors, nbytes):
        """At least one copy; enough copies to exceed 1 GiB in total."""
        r = max(1, math.ceil(ROTATE_BYTES / max(1, nbytes)))
        out = [tensors]
        for _ in range(r - 1):
            out.append(tuple(x.clone() for x in tensors))
        return out

    def time_launches(self, fns, reps, warmup=3, graph=True):
        """Average duration of each launch in fns: `reps` launches of one
        function back to back (f(i) for i = 0..reps-1, so rotating weight
        copies change every launch) between one pair of HIP events.  With
        graph=True the launches are captured once into a HIP graph on a side
        stream and timed as one replay, so a kernel shorter than a Python call
        is not timed at the rate the host can launch it; calls that cannot be
        captured (host synchronisation, allocation) are timed eagerly on
        torch's current stream, which the library launches on."""
        t = self.t
        out = []
        for f in fns:
            for i in range(warmup):
                f(i)
            t.cuda.synchronize()
            us = self._time_graph(f, reps) if graph else None
            if us is None:
                e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(reps):
                    f(i)
                e1.record()
                t.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / reps
            out.append(us)  # microseconds
        return out

    def _time_graph(self, f, reps):
        t = self.t
        # one capture stream for the whole run: the library keeps one
        # workspace per stream, so a fresh stream per timing would hold a new
        # buffer (up to N*K*2 bytes for the split path) each time
        if not hasattr(self, "side"):
            self.side = t.cuda.Stream()
        side = self.side
        # warm up on the capture stream: the library keeps its scratch per
        # stream and must not allocate while the stream is captured
        with t.cuda.stream(side):
            for i in range(2):
                f(i)
        t.cuda.synchronize()
        try:
            g = t.cuda.CUDAGraph()
            with t.cuda.graph(g, stream=side):
                for i in range(reps):
                    f(i)
        except Exception as e:  # not capturable: time eagerly
            log("graph capture failed (%s); timing eagerly" % type(e).__name__)
            t.cuda.synchronize()
            return None
        g.replay()
        t.cuda.synchronize()
        # The mean over three back-to-back replays: the part runs faster for
        # the first millisecond or so after an idle gap than under sustained
        # load, so one short replay would overstate the sustained rate.
        e = [t.cuda.Event(enable_timing=True) for _ in range(4)]
        with t.cuda.stream(side):
            e[0].record(side)
            for r in range(3):
                g.replay()
                e[r + 1].record(side)
        t.cuda.synchronize()
        del g
        return e[0].elapsed_time(e[3]) * 1e3 / (3 * reps)


def fused_source_hash():
    h = hashlib.sha256()
    for f in FUSED_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_from_profile():
    """HBM bytes per launch of the M=1 kernel from the committed counter
    summary, if it was taken on the current fused-kernel source."""
    try:
        text = open(PROFILE_TRAFFIC).read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            k = k.strip()
            if k.startswith("kernel source sha256"):  # "(the files it covers)" may follow
                k = "kernel source sha256"
            fields[k] = v.strip().strip("`")
    if fields.get("kernel source sha256") != fused_source_hash():
        return None
    try:
        return float(fields["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rate(orc, p, M_list, target_s):
    """Algorithmic GB/s of the oracle on a random subset of output columns,
    grown until one pass takes a quarter of the target time; once the whole
    output fits, whole passes are repeated until the target time is reached."""
    N, K = p["N"], p["K"]
    g = synth.rng(123)
    ncols = 16
    while True:
        cols = np.sort(g.choice(N, size=ncols, replace=False))
        t0 = time.perf_counter()
        for M in M_list:
            orc.q4_gemm(p["A"][M][:M], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, BS, cols=cols)
        dt = time.perf_counter() - t0
        if dt >= target_s / 4 or ncols >= N:
            break
        ncols = min(N, int(ncols * max(2.0, (target_s / 4) / max(dt, 1e-3))))
    passes, t_used = 1, dt
    while t_used < target_s and ncols >= N:
        t0 = time.perf_counter()
        for M in M_list:
            orc.q4_gemm(p["A"][M][:M], p["Wpacked"], p["absmax"], p["codebook"], M, N, K, BS, cols=cols)
        t_used += time.perf_counter() - t0
        passes += 1
    total_bytes = passes * sum(q4_bytes(M, N, K) * ncols / N for M in M_list)
    return total_bytes / t_used / 1e9, "%d pass(es) over %d of %d output columns, %.1f s" % (
        passes, ncols, N, t_used)


def cpu_baseline(p, M_list, target_s=10.0):
    """The oracle as it stands, on a bounded sample of the workload, on all
    host cores (the reported value) and on one core."""
    import oracle
    orc = oracle.default()
    cores = os.cpu_count() or 1
    affinity = getattr(os, "sched_getaffinity", None)
    if affinity is not None:
        cores = len(affinity(0))
    orc.set_threads(cores)
    used = orc.max_threads()
    rate_all, sample_all = _oracle_rate(orc, p, M_list, target_s)
    orc.set_threads(1)
    rate_one, sample_one = _oracle_rate(orc, p, M_list, target_s / 2)
    orc.set_threads(used)
    return {
        "value": rate_all,
        "unit": "GB/s",
        "cores": used,
        "kind": "oracle",
        "sample": "fused GEMM M=%s, K=%d, N=%d: %s (algorithmic bytes scaled by the column "
                  "fraction)" % ("/".join(map(str, M_list)), p["K"], p["N"], sample_all),
        "single_thread": {"value": rate_one, "unit": "GB/s", "cores": 1, "sample": sample_one},
        "cpu_model": cpu_model(),
    }


def read_ceiling(d, nbytes, R):
    """Achievable HBM read rate of one launch over nbytes: q4_read_probe (a
    read-only 128-bit stream, default launch shape) over R rotating buffers,
    timed like the per-M kernels."""
    import bit_dequant_skinny_amd as q4
    t = d.t
    nbytes = nbytes // 16 * 16
    bufs = [t.empty(nbytes, dtype=t.uint8, device=d.dev) for _ in range(R)]
    for b in bufs:
        b.fill_(0x5a)
    sink = t.zeros(4, dtype=t.int32, device=d.dev)
    us = d.time_launches([lambda i: q4.q4_read_probe(bufs[i % R], sink)], reps=12 * R)[0]
    del bufs
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"bytes": nbytes, "buffers": R, "us": round(us, 2), "GB/s": round(gbs, 1),
            "frac_of_peak": round(gbs / PEAK_GBS, 4)}


def headline(d, args):
    import bit_dequant_skinny_amd as q4
    t = d.t
    N, K = 28672, 8192
    M_list = args.m
    assert 1 in M_list, "the roofline is taken on the M=1 kernel"
    log("generating the K=%d N=%d workload" % (K, N))
    p = synth.q4_problem(1, N, K, BS, config=1, shape=0)
    p["A"] = {M: synth.activations_bf16(M, K, synth.seed(1, 0, 10 * M + 1)) for M in M_list}
    w = (d.raw(p["Wpacked"]), d.raw(p["absmax"]))
    cb = d.raw(p["codebook"])
    sets = d.copies(w, q4_bytes(1, N, K))
    R = len(sets)
    # The timed path reads the weights in args.layout; the per-M times of the
    # other layout are reported beside them.
    tsets = [(q4.q4_repack_tiles(Wp), am) for Wp, am in sets]
    by_layout = {"rows": sets, "tiles": tsets}
    A = {M: d.bf16(p["A"][M]) for M in M_list}
    C = {M: t.empty((M, N), dtype=t.bfloat16, device=d.dev) for M in M_list}

    def launch(M, i, layout=args.layout):
        Wp, am = by_layout[layout][i % R]
        q4.q4_gemm_skinny(A[M], Wp, am, cb, BS, out=C[M], layout=layout)

    # The timed steps call the C ABI with their arguments prepared once, as a
    # decode loop that holds its buffers does; the binding's argument checks
    # cost several microseconds of host time per call, which left the GPU
    # idle between these ~27 us kernels (reported beside as binding_GB/s).
    L = q4.lib()
    cfn = L.q4_gemm_skinny_tiles if args.layout == "tiles" else L.q4_gemm_skinny_ex
    stream = t.cuda.current_stream().cuda_stream
    prepared = {M: [(A[M].data_ptr(), q4.Q4_DTYPE_BF16, Wp.data_ptr(), am.data_ptr(), cb.data_ptr(),
                     None, M, N, K, BS, C[M].data_ptr(), q4.Q4_DTYPE_BF16, stream, 0)
                    for Wp, am in by_layout[args.layout]] for M in M_list}

    def launch_c(M, i):
        st = cfn(*prepared[M][i % R])
        if st != q4.Q4_OK:
            raise RuntimeError(L.q4_last_error().decode())

    n = 0
    for _ in range(args.warmup):
        for M in M_list:
            launch(M, n)
            n += 1
    t.cuda.synchronize()
    # Per-M kernel times first (back-to-back launches of one M over the
    # rotating weight copies, graph replays between HIP events): besides
    # their own figures they bring the part to its sustained clock before the
    # headline's timed steps (the first tens of milliseconds of load after
    # start-up or idle run well below it: 3.8-4.0 TB/s against 4.7-4.8 TB/s
    # for the same 20 steps once warm).  0.2 s of untimed launches come
    # before the first timing.
    i = 0
    t_end = time.perf_counter() + 0.2
    while time.perf_counter() < t_end:
        for _ in range(8 * R):
            launch_c(M_list[i % len(M_list)], i)
            i += 1
        t.cuda.synchronize()
    # The first graph timing of the process runs slow (measured at M = 1:
    # 30.3 us, then 25.2-26.1 us for the same launches timed again, in any
    # order of M), so one pass over the M values is timed and discarded.
    d.time_launches([lambda i, M=M: launch(M, i) for M in M_list], reps=12 * R)
    # Then four passes over the M values, each M's launch time the mean of
    # its four (one pass alone varied by ~1 us between the M = 1 and M = 4
    # launches, which run the same kernel).
    passes = [d.time_launches([lambda i, M=M: launch(M, i) for M in M_list], reps=12 * R)
              for _ in range(4)]
    per_m_us = {M: sum(p[x] for p in passes) / len(passes) for x, M in enumerate(M_list)}
    # (not with --quick: profiling runs launch one layout only)
    other = "rows" if args.layout == "tiles" else "tiles"
    other_us = {} if args.quick else dict(zip(M_list, d.time_launches(
        [lambda i, M=M: launch(M, i, other) for M in M_list], reps=12 * R)))
    # The K steps captured once into a HIP graph and replayed (reported
    # beside the headline).
    side = t.cuda.Stream()
    with t.cuda.stream(side):
        for M in M_list:
            launch(M, 0)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g, stream=side):
        for _ in range(args.steps):
            for M in M_list:
                launch(M, n)
                n += 1
    # Replayed on the stream it was captured on: one warm-up replay, one
    # timed between synchronisations, then three back to back (sustained).
    with t.cuda.stream(side):
        g.replay()
    t.cuda.synchronize()
    ev = [t.cuda.Event(enable_timing=True) for _ in range(5)]
    t0 = time.perf_counter()
    with t.cuda.stream(side):
        ev[0].record(side)
        g.replay()
        ev[1].record(side)
    t.cuda.synchronize()
    wall = time.perf_counter() - t0
    with t.cuda.stream(side):
        for r in range(3):
            g.replay()
            ev[2 + r].record(side)
    t.cuda.synchronize()
    sustained_ms = ev[1].elapsed_time(ev[4]) / 3
    del g
    # The headline: the K steps issued one call at a time, as a decode loop
    # calls the library, timed by the host clock between synchronisations
    # (and by HIP events on the stream the calls launch on).
    t.cuda.synchronize()
    e_start, e_end = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e_start.record()
    for _ in range(args.steps):
        for M in M_list:
            launch_c(M, n)
            n += 1
    e_end.record()
    t.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    eager_events_s = e_start.elapsed_time(e_end) * 1e-3
    # the same steps through the Python binding
    t.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for M in M_list:
            launch(M, n)
            n += 1
    t.cuda.synchronize()
    binding_wall = time.perf_counter() - t0
    total = args.steps * sum(q4_bytes(M, N, K) for M in M_list)
    per_m = {}
    for M in M_list:
        gbs = q4_bytes(M, N, K) / (per_m_us[M] * 1e-6) / 1e9
        per_m[str(M)] = {"us": round(per_m_us[M], 2), "GB/s": round(gbs, 1),
                         "pct_peak": round(100 * gbs / PEAK_GBS, 1),
                         "path": "fused" if M <= q4.q4_get_crossover_shape(N, K) else "split",
                         other + "_us": round(other_us[M], 2) if other_us else None}
    # The roofline kernel is the M=1 launch, timed as above.
    m1_us = per_m_us[1]
    ach = q4_bytes(1, N, K) / (m1_us * 1e-6) / 1e9
    traffic = traffic_from_profile()
    ceiling = read_ceiling(d, q4_bytes(1, N, K), R)
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_GBS, 4),
            "achievable_read": ceiling,
            "frac_of_achievable_read": round(ach / ceiling["GB/s"], 4),
            "traffic": None if traffic is None else round(traffic / (m1_us * 1e-6) / 1e9, 1),
            "traffic_bytes_per_launch": traffic,
            "kernel": "fused q4 M=1, K=8192, N=28672, %s layout" % args.layout,
            "launch_us": round(m1_us, 2),
            "algorithmic_bytes_per_launch": q4_bytes(1, N, K)}
    out = {
        "metric": METRIC,
        "value": round(total / eager_wall / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(eager_wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "fused 4-bit skinny GEMM, K=8192, N=28672, blocksize 64, "
                               "M=1,2,4,8 per step",
                   "M": M_list, "K": K, "N": N, "blocksize": BS, "weight_copies": R,
                   "weight_layout": args.layout},
        "pct_of_peak": round(100 * total / eager_wall / 1e9 / PEAK_GBS, 1),
        "timed_as": "the K steps issued call by call through the C ABI, host wall clock between "
                    "synchronisations",
        "binding_GB/s": round(total / binding_wall / 1e9, 1),
        "events_GB/s": round(total / eager_events_s / 1e9, 1),
        "graph_replay_GB/s": round(total / wall / 1e9, 1),
        "graph_sustained_GB/s": round(total / (sustained_ms * 1e-3) / 1e9, 1),
        "per_m": per_m,
        "roofline": roof,
    }
    del sets, tsets, by_layout, w
    return out, p, M_list


SWEEP_SHAPES = [  # (K, N, workload index, shape index)
    (5120, 8192, 2, 0), (5120, 5120, 2, 1), (17408, 5120, 2, 2), (8192, 8192, 2, 3),
    (8192, 28672, 1, 0), (2560, 248320, 4, 0)]
SWEEP_M = list(range(1, 17)) + [32, 64, 96, 128, 192, 256, 384, 512]


def crossover_sweep(d, weights):
    """Fused against split (dequantize to bf16 + GEMM) at every M = 1..16 and
    at 32..512 on each shape, weights in the tile layout, rotating copies: the
    measured crossover (the last M up to which the fused path wins) beside the
    library's routing for the shape."""
    import bit_dequant_skinny_amd as q4
    t = d.t
    out = {}
    for K, N, config, shape in SWEEP_SHAPES:
        sets, cb = weights(N, K, config, shape)
        R = len(sets)
        rows = {}
        last_fused_win = 0
        for M in SWEEP_M:
            A = d.bf16(synth.activations_bf16(M, K, synth.seed(config, shape, 10 * M + 1)))
            C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
            fns = []
            for path in ("fused", "split"):
                def f(i, path=path):
                    Wp, am = sets[i % R]
                    q4.q4_gemm_skinny(A, Wp, am, cb, BS, out=C, path=path, layout="tiles")
                fns.append(f)
            uf, us = d.time_launches(fns, reps=max(4, min(24, 2 * R)), warmup=2)
            rows[str(M)] = {"fused_us": round(uf, 2), "split_us": round(us, 2),
                            "fused_GB/s": round(q4_bytes(M, N, K) / (uf * 1e-6) / 1e9, 1)}
            if uf <= us:
                last_fused_win = M
        first_split = next((M for M in SWEEP_M if rows[str(M)]["split_us"] < rows[str(M)]["fused_us"]),
                           None)
        out["K=%d N=%d" % (K, N)] = {
            "us": rows,
            "first M where split beats fused": first_split,
            "last M where fused wins": last_fused_win,
            "library: fused when M <=": q4.q4_get_crossover_shape(N, K),
        }
        log("  K=%d N=%d: split first wins at M=%s (library %d)" % (
            K, N, first_split, q4.q4_get_crossover_shape(N, K)))
    return out


def other_configs(d):
    """Kernel times of the other decode workloads (HIP events, rotated weights)."""
    import bit_dequant_skinny_amd as q4
    t = d.t
    res = {}

    cache = {}

    def q4_weights(N, K, config, shape):
        """Seeded packed weights (row-major and tile layout) rotated over
        >= 1 GiB; one shape is kept at a time."""
        key = (N, K, config, shape)
        if key not in cache:
            cache.clear()
            p = synth.q4_problem(1, N, K, BS, config=config, shape=shape)
            sets = d.copies((d.raw(p["Wpacked"]), d.raw(p["absmax"])), q4_bytes(1, N, K))
            cache[key] = {"rows": sets, "tiles": [(q4.q4_repack_tiles(Wp), am) for Wp, am in sets],
                          "cb": d.raw(p["codebook"])}
        return cache[key]

    def q4_cfg_weights(N, K, config, shape):
        w = q4_weights(N, K, config, shape)
        return w["tiles"], w["cb"]

    def q4_cfg(name, M_list, N, K, config, shape, paths=("auto",), layouts=("rows",)):
        w = q4_weights(N, K, config, shape)
        R = len(w["rows"])
        cases = [(path, lay) for lay in layouts for path in paths]
        cb = w["cb"]
        rows = {}
        for M in M_list:
            A = d.bf16(synth.activations_bf16(M, K, synth.seed(config, shape, 10 * M + 1)))
            C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
            fns = []
            for path, lay in cases:
                def f(i, path=path, lay=lay):
                    Wp, am = w[lay][i % R]
                    q4.q4_gemm_skinny(A, Wp, am, cb, BS, out=C, path=path, layout=lay)
                fns.append(f)
            us = d.time_launches(fns, reps=max(60, min(200, R * 2)))
            for (path, lay), u in zip(cases, us):
                gbs = q4_bytes(M, N, K) / (u * 1e-6) / 1e9
                key = "M=%d %s" % (M, path) + ("" if lay == "rows" else " tiles")
                rows[key] = {"us": round(u, 2), "GB/s": round(gbs, 1),
                             "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
        res[name] = rows
        return rows

    log("C1 GEMV 4096x4096")
    q4_cfg("q4 M=1 K=4096 N=4096", [1], 4096, 4096, 0, 0, layouts=("rows", "tiles"))
    log("fused vs split sweep (crossover): decode layers, FFN, output projection")
    res["crossover sweep"] = crossover_sweep(d, q4_cfg_weights)
    log("C5 large-vocabulary projection, 4-bit (weights of the sweep's last shape)")
    q4_cfg("q4 K=2560 N=248320", [1, 8], 248320, 2560, 4, 0, layouts=("rows", "tiles"))
    cache.clear()
    log("C4 bf16 skinny")
    for shape, N in enumerate([96, 2048, 16384, 31040]):
        K = 2560
        W = d.bf16(synth.bf16_weights(N, K, synth.seed(3, shape, 2)))
        b = d.bf16(synth.bias_bf16(N, synth.seed(3, shape, 3)))
        sets = {"rows": d.copies((W,), bf16_bytes(1, N, K, True))}
        if N % 16 == 0:
            sets["tiles"] = d.copies((q4.bf16_repack_tiles(W),), bf16_bytes(1, N, K, True))
        rows = {}
        for M in range(1, 6):
            A = d.bf16(synth.activations_bf16(M, K, synth.seed(3, shape, 10 * M + 1)))
            C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
            for lay, ws in sets.items():
                def f(i, ws=ws, lay=lay):
                    q4.bf16_gemm_skinny(A, ws[i % len(ws)][0], b, out=C, layout=lay)
                u = d.time_launches([f], reps=max(60, min(200, len(ws) * 2)))[0]
                gbs = bf16_bytes(M, N, K, True) / (u * 1e-6) / 1e9
                rows["M=%d" % M + ("" if lay == "rows" else " tiles")] = {
                    "us": round(u, 2), "GB/s": round(gbs, 1),
                    "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
        res["bf16+bias K=2560 N=%d" % N] = rows
        del sets, W
    log("4-bit path: bias epilogue and other element types, K=8192 N=28672")
    N, K = 28672, 8192
    p = synth.q4_problem(1, N, K, BS, config=1, shape=0)
    sets = d.copies((d.raw(p["Wpacked"]), d.raw(p["absmax"])), q4_bytes(1, N, K))
    cb = d.raw(p["codebook"])
    bias32 = d.raw(synth.bias(N, synth.seed(1, 0, 3), "fp32"))
    rows = {}
    for adt, tdt in (("fp16", t.float16), ("fp32", t.float32)):
        for M in (1, 8):
            a_h = synth.activations(M, K, synth.seed(1, 0, 10 * M + 1), adt)
            A = (d.raw(a_h).view(t.float16) if adt == "fp16" else d.raw(a_h))
            C = t.empty((M, N), dtype=t.float32, device=d.dev)

            def f(i, A=A, C=C):
                Wp, am = sets[i % len(sets)]
                q4.q4_gemm_skinny(A, Wp, am, cb, BS, out=C, bias=bias32, out_dtype=t.float32)
            u = d.time_launches([f], reps=4 * len(sets))[0]
            nbytes = q4_bytes(M, N, K) + (2 if adt == "fp16" else 6) * M * K + 2 * M * N + 4 * N
            gbs = nbytes / (u * 1e-6) / 1e9
            rows["%s A, fp32 C + bias, M=%d" % (adt, M)] = {
                "us": round(u, 2), "GB/s": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
    res["q4 K=8192 N=28672 dtypes+bias"] = rows
    del sets
    log("blockwise quantizer, 28672 x 8192")
    rows = {}
    cbq = q4.q4_codebook_preset("nf4_style")
    for dtn, tdt in (("fp32", t.float32), ("bf16", t.bfloat16)):
        Wq = t.from_numpy(synth.weights_f32(N, K, 85)).to(d.dev).to(tdt)
        outs = (t.empty((N, K // 2), dtype=t.uint8, device=d.dev),
                t.empty((N, K // BS), dtype=t.float32, device=d.dev))
        u = d.time_launches([lambda i: q4.q4_quantize(Wq, cbq, BS, out=outs)], reps=20, graph=False)[0]
        nbytes = N * K * Wq.element_size() + N * K // 2 + 4 * N * K // BS
        gbs = nbytes / (u * 1e-6) / 1e9
        rows["%s W" % dtn] = {"us": round(u, 2), "GB/s": round(gbs, 1),
                              "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
        del Wq, outs
    res["q4_quantize N=28672 K=8192 bs=64"] = rows
    log("C5 large-vocabulary projection, bf16")
    K, N = 2560, 248320
    W = d.bf16(synth.bf16_weights(N, K, synth.seed(4, 1, 2)))
    Ws = {"rows": W, "tiles": q4.bf16_repack_tiles(W)}
    rows = {}
    for M in range(1, 6):
        A = d.bf16(synth.activations_bf16(M, K, synth.seed(4, 1, 10 * M + 1)))
        C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
        for lay, Wl in Ws.items():
            u = d.time_launches([lambda i, Wl=Wl, lay=lay: q4.bf16_gemm_skinny(
                A, Wl, None, out=C, layout=lay)], reps=20)[0]
            gbs = bf16_bytes(M, N, K, False) / (u * 1e-6) / 1e9
            rows["M=%d" % M + ("" if lay == "rows" else " tiles")] = {
                "us": round(u, 2), "GB/s": round(gbs, 1),
                "pct_peak": round(100 * gbs / PEAK_GBS, 1)}
    res["bf16 K=2560 N=248320"] = rows
    del W, Ws
    res["copy probe 1 GiB (read+write)"] = copy_probe(d)
    res["read probe 1 GiB"] = read_ceiling(d, 1 << 30, 1)
    return res


def copy_probe(d, nbytes=1 << 30):
    """The achievable copy rate with the same 128-bit loads (context for % of
    peak, and the known-size kernel the HBM byte counters are scaled by)."""
    import bit_dequant_skinny_amd as q4
    src = d.t.empty(nbytes, dtype=d.t.uint8, device=d.dev)
    dst = d.t.empty_like(src)
    u = d.time_launches([lambda i: q4.q4_copy_probe(src, dst)], reps=20)[0]
    return {"bytes_read": nbytes, "bytes_written": nbytes, "us": round(u, 1),
            "GB/s": round(2 * nbytes / (u * 1e-6) / 1e9, 1)}


def profile_case(d, which, launches=12):
    """A few launches of one call for counter and trace runs: the split path
    (dequantize + bf16 GEMM) on the FFN at M = 16 and 256, or the bf16 skinny
    GEMM on the 248320 x 2560 projection at M = 1 (row-major or tile layout),
    or the fused skinny kernel with K parts on 5120 x 17408 at M = 1 or 32;
    weights rotate as in the timed runs."""
    import bit_dequant_skinny_amd as q4
    t = d.t
    if which in ("split16", "split256"):
        M = 16 if which == "split16" else 256
        N, K = 28672, 8192
        p = synth.q4_problem(1, N, K, BS, config=1, shape=0)
        sets = d.copies((d.raw(p["Wpacked"]), d.raw(p["absmax"])), q4_bytes(1, N, K))
        cb = d.raw(p["codebook"])
        A = d.bf16(synth.activations_bf16(M, K, synth.seed(1, 0, 10 * M + 1)))
        C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
        for i in range(launches):
            Wp, am = sets[i % len(sets)]
            q4.q4_gemm_skinny(A, Wp, am, cb, BS, out=C, path="split")
    elif which in ("kparts", "kparts32"):
        # the skinny kernel with K split over workgroups, then the part sum
        # (kparts32: 32 token rows, two token blocks per pass)
        N, K, M = 5120, 17408, 32 if which == "kparts32" else 1
        p = synth.q4_problem(1, N, K, BS, config=2, shape=2)
        sets = d.copies((q4.q4_repack_tiles(d.raw(p["Wpacked"])), d.raw(p["absmax"])),
                        q4_bytes(1, N, K))
        cb = d.raw(p["codebook"])
        A = d.bf16(synth.activations_bf16(M, K, synth.seed(2, 2, 10 * M + 1)))
        C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
        for i in range(launches):
            Wt, am = sets[i % len(sets)]
            q4.q4_gemm_skinny(A, Wt, am, cb, BS, out=C, layout="tiles")
    elif which in ("bf16c5", "bf16c5tiles"):
        N, K, M = 248320, 2560, 1
        W = d.bf16(synth.bf16_weights(N, K, synth.seed(4, 1, 2)))
        lay = "tiles" if which == "bf16c5tiles" else "rows"
        if lay == "tiles":
            W = q4.bf16_repack_tiles(W)
        A = d.bf16(synth.activations_bf16(M, K, synth.seed(4, 1, 10 * M + 1)))
        C = t.empty((M, N), dtype=t.bfloat16, device=d.dev)
        for _ in range(launches):
            q4.bf16_gemm_skinny(A, W, None, out=C, layout=lay)
    else:
        raise ValueError(which)
    t.cuda.synchronize()
    print(json.dumps({"profile_case": which, "launches": launches}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--m", type=int, nargs="+", default=[1, 2, 4, 8],
                    help="token rows per step (profiling runs use --m 1)")
    ap.add_argument("--layout", choices=("tiles", "rows"), default="tiles",
                    help="packed-weight layout of the timed step (q4_repack_tiles or row-major)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the 1 GiB copy kernel (counter calibration)")
    ap.add_argument("--profile-case",
                    choices=("split16", "split256", "bf16c5", "bf16c5tiles", "kparts", "kparts32"),
                    help="only run a few launches of one call (for rocprofv3 runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    d = Dev()
    assert d.t.cuda.is_available(), "bench.py needs an MI355X"
    if args.copy_probe:
        print(json.dumps({"copy probe 1 GiB (read+write)": copy_probe(d)}), flush=True)
        return
    if args.profile_case:
        profile_case(d, args.profile_case)
        return
    out, p, M_list = headline(d, args)
    log("headline: %.1f GB/s" % out["value"])
    if not args.quick:
        out["configs"] = other_configs(d)
    if not args.no_cpu:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(p, M_list)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
