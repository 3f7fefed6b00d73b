#!/usr/bin/env python3
"""Throughput of the quantized matvec / small-M matmul hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--detail-out FILE]

A step is one pass over every call of the workload with one set of inputs
already resident in HBM.  The default workload is the 4-bit, group-size-64,
bfloat16 path the metric is quoted on:

* qmv, M = 1, over (N, K) in {5120x5120, 14336x5120, 5120x14336, 27648x5120};
* the policy-dispatched qmm (qmv, unsplit qmm_t or split-K + accumulate) over
  (K, N, M) in {(2048, 2048, 22), (4096, 4096, 16), (256, 4096, 16),
  (10752, 2048, 85), (14336, 4096, 33), (17408, 5120, 56)}.

Inputs are drawn on the device (seeded).  R distinct input sets rotate
from step to step so that the working set between two uses of a set exceeds
the 256 MB Infinity Cache three times over and weights come from HBM.  Each
set's step is captured once in a HIP graph and replayed, so host launch cost
is not timed.  `value` is algorithmic bytes moved per second over the K timed
steps (GB/s); per-call microseconds come from HIP events around graphs that
replay one call over the rotating sets.

One JSON line is printed on stdout.  `--gpus` above 1 is refused: the
benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16/f16 MFMA, published
MALL_BYTES = 256 * 2 ** 20
METRIC = "µs/call & effective HBM GB/s (% roofline), 4-bit affine gs=64 qmv/qmm, bf16"

F32, F16, BF16 = 0, 1, 2
DT_NAME = {F32: "f32", F16: "f16", BF16: "bf16"}


def affine(route, M, N, K, dt=BF16, bits=4, gs=64, B=1, E=1, sorted_idx=False):
    c = {"kind": "affine", "route": route, "M": M, "N": N, "K": K, "bits": bits, "gs": gs, "dtype": dt, "B": B,
         "E": E}
    if sorted_idx:   # gather with the problems ordered by weight matrix (qmx_qmm_gather_sorted)
        c["sorted"] = True
    return c


def block(kind, N, K):
    return {"kind": kind, "route": kind, "M": 1, "N": N, "K": K, "dtype": F32}


QMV_SHAPES = [(5120, 5120), (14336, 5120), (5120, 14336), (27648, 5120)]
QMM_SHAPES = [(2048, 2048, 22), (4096, 4096, 16), (256, 4096, 16), (10752, 2048, 85), (14336, 4096, 33),
              (17408, 5120, 56)]

WORKLOADS = {
    "qmv_qmm_4bit_gs64_bf16": [affine("qmv", 1, n, k) for n, k in QMV_SHAPES]
    + [affine("qmm", m, n, k) for k, n, m in QMM_SHAPES],
    # the same calls at the other code widths of the staged loader (1-6 and 8 bits)
    **{f"qmv_qmm_{b}bit_gs64_bf16": [affine("qmv", 1, n, k, bits=b) for n, k in QMV_SHAPES]
       + [affine("qmm", m, n, k, bits=b) for k, n, m in QMM_SHAPES] for b in (1, 2, 3, 5, 6, 8)},
    "qmv_4bit_gs64_bf16": [affine("qmv", 1, n, k) for n, k in QMV_SHAPES],
    "qmv_4bit_gs64_f16": [affine("qmv", 1, n, k, F16) for n, k in QMV_SHAPES],
    "qmv_4bit_gs64_f32": [affine("qmv", 1, n, k, F32) for n, k in QMV_SHAPES],
    "qmv_4bit_gs64_f32_4096": [affine("qmv", 1, 4096, 4096, F32)],
    # small decode batches (M = 2..7 rows of x share each weight read)
    "qmv_small_m_4bit_gs64_bf16": [affine("qmv", m, n, k) for m in (2, 4, 7) for n, k in ((4096, 4096), (14336, 5120))],
    "qmm_4bit_gs64_bf16": [affine("qmm", m, n, k) for k, n, m in QMM_SHAPES],
    "qmm_control_4096_m512": [affine("qmm", 512, 4096, 4096)],
    # the compute-bound regime: larger M on the same weights (illustrative sizes)
    "qmm_large_m_4bit_gs64_bf16": [affine("qmm", m, n, k) for k, n, m in
                                   ((4096, 4096, 512), (4096, 4096, 1024), (4096, 4096, 2048), (4096, 14336, 1024))],
    # batches of independent problems, each with its own weights (qmx_qmm_batched):
    # illustrative shapes of the config-1 size class, not taken from the pages
    "batched_4bit_gs64_bf16": [affine("batched", 1, 4096, 4096, B=8), affine("batched", 16, 2048, 4096, B=8),
                               affine("batched", 56, 2048, 5120, B=4)],
    # B problems gathering from E weight matrices (qmx_qmm_gather; every matrix is used, each by
    # B/E problems, in random order; then the same picks ordered by matrix through
    # qmx_qmm_gather_sorted), illustrative shapes as above
    "gather_4bit_gs64_bf16": [affine("gather", 1, 2048, 4096, B=16, E=8), affine("gather", 16, 2048, 4096, B=16, E=8),
                              affine("gather", 1, 2048, 4096, B=16, E=8, sorted_idx=True)],
    "q8_0_14336x5120": [block("q8_0", 14336, 5120)],
    "q8_i8_14336x5120": [block("q8_i8", 14336, 5120)],
    "q4_k_14336x5120": [block("q4_k", 14336, 5120)],
}
DEFAULT_WORKLOAD = "qmv_qmm_4bit_gs64_bf16"


def call_name(c):
    if c["kind"] == "affine":
        head = c["route"] if c.get("B", 1) == 1 else f"{c['route']}{c['B']}"
        if c["route"] == "gather":
            head = head.replace("gather", "gathersorted" if c.get("sorted") else "gather") + f"of{c['E']}"
        return f"{head}_M{c['M']}_N{c['N']}_K{c['K']}_b{c['bits']}_gs{c['gs']}_{DT_NAME[c['dtype']]}"
    return f"{c['kind']}_N{c['N']}_K{c['K']}"


def alg_bytes(c):
    """Bytes the method must move once (weights, scales/biases, x, out)."""
    M, N, K = c["M"], c["N"], c["K"]
    if c["kind"] == "q8_0":
        return N * (K // 32) * 36 + 4 * K + 4 * N
    if c["kind"] == "q4_k":
        return N * (K // 256) * 144 + 4 * K + 4 * N
    if c["kind"] == "q8_i8":   # int8 weights, float32 block scales, int8 x, float32 out
        return N * K + N * (K // 32) * 4 + K + 4 * N
    e = 4 if c["dtype"] == F32 else 2
    G = K // c["gs"]
    if c["route"] == "gather":   # each of the E weight matrices is needed once; x and out per problem
        return c["E"] * (N * K * c["bits"] // 8 + 2 * N * G * e) + c["B"] * (M * K * e + M * N * e)
    return c.get("B", 1) * (N * K * c["bits"] // 8 + 2 * N * G * e + M * K * e + M * N * e)


def flops(c):
    return 2 * c.get("B", 1) * c["M"] * c["N"] * c["K"]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="one of: " + ", ".join(sorted(WORKLOADS)) + ", or only:<call name>")
    ap.add_argument("--reps", type=int, default=20, help="replays per per-call timing graph")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail-out", default=None, help="write per-call details as JSON here")
    ap.add_argument("--seed", type=int, default=20261202)
    return ap.parse_args(argv)


def resolve_workload(name):
    if name.startswith("only:"):
        want = name[5:]
        for calls in WORKLOADS.values():
            for c in calls:
                if call_name(c) == want:
                    return [c]
        raise SystemExit(f"unknown call {want}")
    if name not in WORKLOADS:
        raise SystemExit(f"unknown workload {name}; choose from {sorted(WORKLOADS)}")
    return WORKLOADS[name]


# ---------------------------------------------------------------- device inputs
def make_inputs(c, seed, dev):
    import torch

    import matmul_affine_qmv_amd as qmx
    import qmx_inputs as qi
    if c["kind"] == "affine" and c["route"] == "gather":
        parts = [qi.affine_case_torch(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"], seed + i, dev)
                 for i in range(c["E"])]
        d = {k: torch.stack([p[k] for p in parts]) for k in ("w", "scales", "biases")}
        d["x"] = torch.stack([qi.affine_case_torch(c["M"], 32, c["K"], 4, c["gs"], c["dtype"], seed + 1000 + i,
                                                   dev)["x"] for i in range(c["B"])])
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        wi = torch.randperm(c["B"], generator=g) % c["E"]
        if c.get("sorted"):
            wi = torch.sort(wi).values
        d["w_index"] = wi.to(torch.int32).to(dev)
        d["out"] = torch.empty((c["B"], c["M"], c["N"]), dtype=d["x"].dtype, device=dev)
        need = qmx.lib().qmx_qmm_gather_workspace_bytes(c["B"], c["B"], c["M"], c["N"], c["K"], c["bits"], c["gs"],
                                                         c["dtype"], d["x"].data_ptr(), c["M"] * c["K"], c["K"])
        d["ws"] = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev) if need else None
        return d
    if c["kind"] == "affine" and c["route"] == "batched":
        parts = [qi.affine_case_torch(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"], seed + i, dev)
                 for i in range(c["B"])]
        d = {k: torch.stack([p[k] for p in parts]) for k in ("w", "scales", "biases", "x")}
        d["out"] = torch.empty((c["B"], c["M"], c["N"]), dtype=d["x"].dtype, device=dev)
        need = qmx.lib().qmx_qmm_batched_workspace_bytes(c["B"], c["M"], c["N"], c["K"], c["bits"], c["gs"],
                                                          c["dtype"], d["x"].data_ptr(), c["M"] * c["K"], c["K"])
        d["ws"] = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev) if need else None
        return d
    if c["kind"] == "affine":
        d = qi.affine_case_torch(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"], seed, dev)
        d["out"] = torch.empty((c["M"], c["N"]), dtype=d["x"].dtype, device=dev)
        need = 0
        if c["route"] == "qmm":
            need = qmx.qmm_workspace_bytes(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"])
        d["ws"] = torch.empty(max(1, need // 4), dtype=torch.float32, device=dev) if need else None
        return d
    if c["kind"] == "q8_i8":
        d = qi.q8_i8_case_torch(c["N"], c["K"], seed, dev)
        d["out"] = torch.empty(c["N"], dtype=torch.float32, device=dev)
        return d
    gen = qi.q8_0_case_torch if c["kind"] == "q8_0" else qi.q4_k_case_torch
    d = gen(c["N"], c["K"], seed, dev)
    d["out"] = torch.empty(c["N"], dtype=torch.float32, device=dev)
    return d


def footprint(c, d):
    keys = ("w", "scales", "biases", "x", "blocks", "wq", "xq", "wd")
    return sum(d[k].numel() * d[k].element_size() for k in keys if k in d)


def launch(c, d):
    import matmul_affine_qmv_amd as qmx
    if c["kind"] == "q8_0":
        return qmx.matvec_q8_0(d["blocks"], d["x"], d["out"])
    if c["kind"] == "q4_k":
        return qmx.matvec_q4_k(d["blocks"], d["x"], d["out"])
    if c["kind"] == "q8_i8":
        return qmx.matvec_q8_i8(d["wq"], d["xq"], d["wd"], d["out"])
    kw = dict(bits=c["bits"], group_size=c["gs"])
    if c["route"] == "gather":
        return qmx.gather_qmm(d["w"], d["scales"], d["biases"], d["x"], d["w_index"], None, d["out"],
                              workspace=d["ws"], sorted_indices=c.get("sorted", False), **kw)
    if c["route"] == "batched":
        return qmx.qmm_batched(d["w"], d["scales"], d["biases"], d["x"], d["out"], workspace=d["ws"], **kw)
    if c["route"] == "qmv":
        return qmx.qmv(d["w"], d["scales"], d["biases"], d["x"], d["out"], **kw)
    return qmx.qmm(d["w"], d["scales"], d["biases"], d["x"], d["out"], workspace=d["ws"], **kw)


# ---------------------------------------------------------------- timing
def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graphs(graphs, steps):
    """Replay graphs round-robin `steps` times; returns (wall seconds, GPU event ms)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(steps):
        graphs[k % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, start.elapsed_time(end)


def per_call_us(c, sets, idx, reps):
    """Average µs per launch of call `idx`: a graph launches it once per rotating
    set; the graph is replayed `reps` times between two HIP events."""
    g = capture(lambda: [launch(c, s[idx]) for s in sets])
    time_graphs([g], 3)   # warm-up: the GPU idles while the host captures
    _, ms = time_graphs([g], reps)
    return 1000.0 * ms / (reps * len(sets))


def per_kernel_us(fn, sets, idx, reps):
    """Average µs per launch of one kernel: a graph launches it once per rotating
    set; the graph is replayed `reps` times between two HIP events on the
    stream the kernels run on."""
    g = capture(lambda: [fn(s[idx]) for s in sets])
    time_graphs([g], 3)   # warm-up: the GPU idles while the host captures
    _, ms = time_graphs([g], reps)
    return 1000.0 * ms / (reps * len(sets))


def roofline_for(c, us, nbytes=None, nflops=None, matrix=None):
    """Roofline of one launch: HBM-bound unless the bf16/f16 MFMA time at the
    published peak exceeds the HBM time at the published peak."""
    b = alg_bytes(c) if nbytes is None else nbytes
    f = flops(c) if nflops is None else nflops
    if matrix is None:
        matrix = c["kind"] == "affine" and c["route"] == "qmm" and c["M"] >= 8 and c["dtype"] != F32
    t_hbm = b / (HBM_PEAK_GBS * 1e9)
    t_mfma = f / (MFMA_BF16_TFLOPS * 1e12) if matrix else 0.0
    s = us * 1e-6
    if t_mfma > t_hbm:
        ach = f / s / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / MFMA_BF16_TFLOPS}
    ach = b / s / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS}


def kernels_of(c, route, splits):
    """The kernels one call launches, each as (label, launcher over an input set,
    algorithmic bytes per launch, flops per launch, on the matrix cores)."""
    import matmul_affine_qmv_amd as qmx
    if c["kind"] == "affine" and c["route"] in ("batched", "gather"):
        # one launch sequence for the whole batch, timed as a whole
        return [(f"qmm_{c['route']} (whole call)", lambda d, c=c: launch(c, d), alg_bytes(c), flops(c), c["M"] >= 8)]
    if c["kind"] != "affine" or route != "qmm_t_splitk":
        label = {"qmv": "qmv_kernel", "qmm_t": "qmm_t_kernel", "q8_0": "q8_0_kernel",
                 "q4_k": "q4_k_kernel", "q8_i8": "q8_i8_kernel"}[route if c["kind"] == "affine" else c["kind"]]
        return [(label, lambda d, c=c: launch(c, d), alg_bytes(c), flops(c), route == "qmm_t")]
    M, N, K, e = c["M"], c["N"], c["K"], 2
    parts = splits * M * N * 4
    inputs = alg_bytes(c) - M * N * e
    kw = dict(bits=c["bits"], group_size=c["gs"], splits=splits)
    return [
        ("qmm_t_kernel (split-K partials)",
         lambda d: qmx.qmm_t_partials(d["w"], d["scales"], d["biases"], d["x"], workspace=d["ws"], **kw),
         inputs + parts, flops(c), True),
        ("splitk_accum_kernel", lambda d: qmx.splitk_accumulate(d["ws"], d["out"], splits), parts + M * N * e,
         0, False),
    ]


def stored_traffic(call, label):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel, if a
    summary under profiles/ matches the current kernel sources; else None."""
    import glob

    from matmul_affine_qmv_amd import traffic
    digest = traffic.source_digest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))):
        try:
            with open(path) as f:
                t = json.load(f)
        except (OSError, ValueError):
            continue
        if t.get("call") == call and t.get("kernel_label") == label and t.get("source_sha256") == digest:
            return t["traffic_bytes_per_launch"], os.path.relpath(path, ROOT)
    return None, None


# ---------------------------------------------------------------- oracle baseline
def cpu_baseline(calls, sets, target_s):
    """Time the float64 oracle on a column sample of every call (set 0) and check
    the GPU outputs of those columns against it."""
    import numpy as np

    import matmul_affine_qmv_amd as qmx
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare

    orc = oracle.load()
    host = []
    for i, c in enumerate(calls):
        d = sets[0][i]
        if c.get("B", 1) > 1:   # a batch: the oracle takes its first problem
            wi = int(d["w_index"][0]) if "w_index" in d else 0
            d = {k: v[wi if k in ("w", "scales", "biases") else 0] for k, v in d.items()
                 if k in ("w", "scales", "biases", "x", "out")}
        h = {k: qmx.tensor_bits(d[k]) for k in ("w", "scales", "biases", "x", "blocks", "wq", "xq", "wd", "out")
             if k in d}
        for k in ("w", "blocks", "wq", "xq"):
            if k in h:
                h[k] = h[k].view(np.uint32)
        host.append(h)
    macs = [c["M"] * c["N"] * c["K"] for c in calls]
    # probe the oracle's rate on a small slice of the first call
    rate = None
    frac = 1.0
    done_bytes, done_s, worst = 0.0, 0.0, None
    for i, c in enumerate(calls):
        h = host[i]
        if rate is not None:
            frac = min(1.0, target_s * rate / max(1, sum(macs)))
        ncols = max(8, int(round(c["N"] * frac)))
        cols = np.linspace(0, c["N"] - 1, num=min(ncols, c["N"]), dtype=np.int64).astype(np.int32)
        t0 = time.perf_counter()
        if c["kind"] == "affine":
            ref = orc.affine(h["w"], h["scales"], h["biases"], c["dtype"], h["x"], c["dtype"], c["M"], c["N"],
                             c["K"], c["bits"], c["gs"], cols=cols)
        elif c["kind"] == "q8_0":
            ref = orc.q8_0(h["blocks"], h["x"], c["N"], c["K"], rows=cols)
        elif c["kind"] == "q8_i8":
            ref = orc.q8_i8(h["wq"], h["xq"], h["wd"], c["N"], c["K"], rows=cols)
        else:
            ref = orc.q4_k(h["blocks"], h["x"], c["N"], c["K"], rows=cols)
        dt_s = time.perf_counter() - t0
        f_done = len(cols) / c["N"]
        done_bytes += alg_bytes(dict(c, B=1, E=1, route="qmm")) * f_done
        done_s += dt_s
        if rate is None:
            rate = c["M"] * len(cols) * c["K"] / max(dt_s, 1e-6)
        import qmx_inputs as qi
        got = qi.storage_to_f64(h["out"], c["dtype"])
        got = got[:, cols] if got.ndim == 2 else got[cols]
        m = compare(got, ref, c["dtype"], orc)
        if worst is None or m["rel_l2"] / m["rel_gate"] > worst[1]:
            worst = (call_name(c), m["rel_l2"] / m["rel_gate"], m["ok"])
        if not m["ok"]:
            worst = (call_name(c), m["rel_l2"] / m["rel_gate"], False)
            break
    return {
        "value": done_bytes / done_s / 1e9 if done_s > 0 else None,
        "unit": "GB/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "sample": (f"float64 C oracle (OpenMP) on an evenly spaced sample of output columns of every call "
                   f"(about {100 * frac:.1f}% of columns after the first call), input set 0; "
                   f"bytes scaled by the sampled fraction; {done_s:.1f} s wall time on {orc.num_threads()} threads"),
        "parity_ok": bool(worst[2]) if worst else None,
        "parity_worst": {"call": worst[0], "rel_l2_over_gate": worst[1]} if worst else None,
    }


# ---------------------------------------------------------------- main
def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the benchmark runs on exactly one GPU "
              f"(the hot path would shard across GPUs by output rows of W)", file=sys.stderr)
        return 2
    import torch

    import matmul_affine_qmv_amd as qmx
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    qmx.lib()
    dev = "cuda:0"
    calls = resolve_workload(args.workload)

    # input sets: at least 3x the MALL is touched between two uses of a set
    set0 = [make_inputs(c, args.seed + 7919 * i, dev) for i, c in enumerate(calls)]
    per_set = sum(footprint(c, d) for c, d in zip(calls, set0))
    nsets = max(3, math.ceil(3 * MALL_BYTES / per_set))
    sets = [set0] + [[make_inputs(c, args.seed + 104729 * r + 7919 * i, dev) for i, c in enumerate(calls)]
                     for r in range(1, nsets)]
    torch.cuda.synchronize()

    # eager warm-up (loads code objects, caches the CU count), then capture one graph per set
    for s in sets:
        for c, d in zip(calls, s):
            launch(c, d)
    torch.cuda.synchronize()
    graphs = [capture(lambda s=s: [launch(c, d) for c, d in zip(calls, s)]) for s in sets]
    time_graphs(graphs, max(args.warmup, 1) * len(graphs))

    wall, gpu_ms = time_graphs(graphs, args.steps)
    step_bytes = sum(alg_bytes(c) for c in calls)
    step_flops = sum(flops(c) for c in calls)
    value = args.steps * step_bytes / wall / 1e9

    details, kernels = [], []
    for i, c in enumerate(calls):
        us = per_call_us(c, sets, i, args.reps)
        route, splits = c["route"], 1
        if c["kind"] == "affine" and route == "qmm":
            route, splits = qmx.plan(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"])
        elif c["kind"] == "affine" and route in ("batched", "gather"):
            route, splits = qmx.plan_batched(c["B"], c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"])
        shown = route if route != "qmm_t_splitk" else f"qmm_t_splitk{splits}"
        details.append({"call": call_name(c), "route": shown, "us": us, "alg_bytes": alg_bytes(c),
                        "gbs": alg_bytes(c) / us / 1e3, "hbm_frac": alg_bytes(c) / us / 1e3 / HBM_PEAK_GBS,
                        "tflops": flops(c) / us / 1e6, "roofline": roofline_for(c, us)})
        for label, fn, kb, kf, matrix in kernels_of(c, route if c["kind"] == "affine" else c["kind"], splits):
            kus = per_kernel_us(fn, sets, i, args.reps)
            kernels.append({"call": call_name(c), "kernel": label, "us": kus, "alg_bytes": kb, "flops": kf,
                            "roofline": roofline_for(c, kus, kb, kf, matrix)})
    dom = max(kernels, key=lambda k: k["us"])
    roof = dict(dom["roofline"])
    traffic, traffic_src = stored_traffic(dom["call"], dom["kernel"])
    roof.update({"kernel": dom["kernel"], "call": dom["call"], "us_per_launch": dom["us"],
                 "alg_bytes_per_launch": dom["alg_bytes"], "flops_per_launch": dom["flops"],
                 "traffic": traffic, "traffic_source": traffic_src})

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(calls, sets, args.cpu_seconds)

    line = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else
        f"µs/call & effective HBM GB/s (% roofline), workload {args.workload}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1000 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if all(c["dtype"] == BF16 for c in calls) else "+".join(
            sorted({DT_NAME[c["dtype"]] for c in calls})),
        "data": "synthetic",
        "config": {"workload": args.workload, "calls": len(calls), "rotating_sets": nsets,
                   "set_bytes": per_set, "step_alg_bytes": step_bytes, "step_flops": step_flops,
                   "graph_replay": True, "gpu_ms_per_step": round(gpu_ms / args.steps, 4)},
        "us_per_call": {d["call"]: round(d["us"], 3) for d in details},
        "hbm_frac_per_call": {d["call"]: round(d["hbm_frac"], 4) for d in details},
        "routes": {d["call"]: d["route"] for d in details},
        "us_per_kernel": {f"{k['call']}:{k['kernel']}": round(k["us"], 3) for k in kernels},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump({"line": line, "details": details, "kernels": kernels}, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
