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

Whole steps: R distinct input sets rotate from step to step so that at least
three times the 256 MB Infinity Cache is touched between two uses of a set;
each set's step is captured once in a HIP graph and replayed (no host launch
cost); `value` is algorithmic bytes per second over the K timed steps.  The
calls' split-K workspaces (scratch, not inputs) are one buffer shared by all
calls and sets.  Before the timed steps come the W warm-up steps of every set
and then more untimed replays until the GPU has been busy for 50 ms, since
its clock ramps up over the first milliseconds of load.

Per call and per kernel: every call gets its own rotation of distinct input
sets totalling at least 512 MiB (twice the Infinity Cache), so no call is
served from it; a graph launches the call (or one of its kernels) once per
set; after 20 warm-up calls, at least 200 calls are timed between two HIP
events on the stream the kernels run on, 5 times, and the median is kept.

Calibration kernels (libqmx_calib.so) give what the GPU reaches for a plain
streaming read of each call's bytes and for back-to-back bf16 matrix-core
instructions, next to the published peaks.

One JSON line is printed on stdout.  `--gpus` above 1 is refused: the
benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16/f16 MFMA, published
MALL_BYTES = 256 * 2 ** 20
ROTATION_BYTES = 512 * 2 ** 20  # per-call rotation: twice the Infinity Cache
CALLS_PER_REPEAT = 200
REPEATS = 5
WARMUP_CALLS = 20
METRIC = "µs/call & effective HBM GB/s (% roofline), 4-bit affine gs=64 qmv/qmm, bf16"

F32, F16, BF16 = 0, 1, 2
DT_NAME = {F32: "f32", F16: "f16", BF16: "bf16"}


def affine(route, M, N, K, dt=BF16, bits=4, gs=64, B=1, E=1, sorted_idx=False, splits=None):
    c = {"kind": "affine", "route": route, "M": M, "N": N, "K": K, "bits": bits, "gs": gs, "dtype": dt, "B": B,
         "E": E}
    if sorted_idx:   # gather with the problems ordered by weight matrix (qmx_qmm_gather_sorted)
        c["sorted"] = True
    if splits is not None:   # route "splitk": qmx_qmm_t_splitk at a forced split count
        c["splits"] = splits
    return c


def block(kind, N, K):
    return {"kind": kind, "route": kind, "M": 1, "N": N, "K": K, "dtype": F32}


QMV_SHAPES = [(5120, 5120), (14336, 5120), (5120, 14336), (27648, 5120)]
QMM_SHAPES = [(2048, 2048, 22), (4096, 4096, 16), (256, 4096, 16), (10752, 2048, 85), (14336, 4096, 33),
              (17408, 5120, 56)]
SWEEP_M = (1, 8, 33, 128, 257)

WORKLOADS = {
    "qmv_qmm_4bit_gs64_bf16": [affine("qmv", 1, n, k) for n, k in QMV_SHAPES]
    + [affine("qmm", m, n, k) for k, n, m in QMM_SHAPES],
    # the same calls at the other code widths of the staged loader (1-6 and 8 bits)
    **{f"qmv_qmm_{b}bit_gs64_bf16": [affine("qmv", 1, n, k, bits=b) for n, k in QMV_SHAPES]
       + [affine("qmm", m, n, k, bits=b) for k, n, m in QMM_SHAPES] for b in (1, 2, 3, 5, 6, 8)},
    "qmv_4bit_gs64_bf16": [affine("qmv", 1, n, k) for n, k in QMV_SHAPES],
    "qmv_4bit_gs64_f16": [affine("qmv", 1, n, k, F16) for n, k in QMV_SHAPES],
    "qmv_4bit_gs64_f32": [affine("qmv", 1, n, k, F32) for n, k in QMV_SHAPES],
    # one float32 matvec, 4096 x 4096
    "qmv_4bit_gs64_f32_4096": [affine("qmv", 1, 4096, 4096, F32)],
    # small decode batches (M = 2..7 rows of x share each weight read)
    "qmv_small_m_4bit_gs64_bf16": [affine("qmv", m, n, k) for m in (2, 4, 7) for n, k in ((4096, 4096), (14336, 5120))],
    "qmm_4bit_gs64_bf16": [affine("qmm", m, n, k) for k, n, m in QMM_SHAPES],
    # the small-M shapes at every split count of 2-4 that keeps 256 columns per partition,
    # beside the unsplit kernel
    "qmm_splits_4bit_gs64_bf16": [affine("qmm_t", m, n, k) for k, n, m in QMM_SHAPES]
    + [affine("splitk", m, n, k, splits=s) for k, n, m in QMM_SHAPES for s in (2, 3, 4) if k >= 512 and k // 256 >= s],
    "qmm_control_4096_m512": [affine("qmm", 512, 4096, 4096)],
    # the compute-bound regime: larger M on the same weights (illustrative sizes)
    "qmm_large_m_4bit_gs64_bf16": [affine("qmm", m, n, k) for k, n, m in
                                   ((4096, 4096, 512), (4096, 4096, 1024), (4096, 4096, 2048), (4096, 14336, 1024))],
    # quantization sweep: widths 2/4/8, group sizes 32/64/128, 16-bit activations, M = 1..257, N = K = 4096
    "sweep_4096": [affine("qmm", m, 4096, 4096, dt, bits=b, gs=g)
                   for b in (2, 4, 8) for g in (32, 64, 128) for dt in (F16, BF16) for m in SWEEP_M],
    # batches of independent problems, each with its own weights (qmx_qmm_batched):
    # illustrative shapes of the 4096 x 4096 size class, not taken from the pages
    "batched_4bit_gs64_bf16": [affine("batched", 1, 4096, 4096, B=8), affine("batched", 16, 2048, 4096, B=8),
                               affine("batched", 56, 2048, 5120, B=4)],
    # B problems gathering from E weight matrices (qmx_qmm_gather; every matrix is used, each by
    # B/E problems, in random order; then the same picks ordered by matrix through
    # qmx_qmm_gather_sorted), illustrative shapes as above
    "gather_4bit_gs64_bf16": [affine("gather", 1, 2048, 4096, B=16, E=8), affine("gather", 16, 2048, 4096, B=16, E=8),
                              affine("gather", 1, 2048, 4096, B=16, E=8, sorted_idx=True)],
    # M = 2..7 on the vector route, the matrix routes unsplit and split 2/4/8, and the policy's pick
    "route_small_m_4bit_gs64_bf16": [c for n, k in ((4096, 4096), (14336, 5120), (5120, 5120), (27648, 5120),
                                                    (4096, 14336))
                                     for m in (2, 4, 5, 7)
                                     for c in [affine("qmm", m, n, k), affine("qmv", m, n, k), affine("qmm_t", m, n, k)]
                                     + [affine("splitk", m, n, k, splits=s) for s in (2, 4, 8)
                                        if k // 256 >= s and (n + 127) // 128 * s <= 512]],
    # group size 32 at M = 8..32: the unsplit narrow tiles against the split plans, and the policy's pick
    "route_narrow_gs32_4bit_bf16": [c for n, k in ((4096, 4096), (2048, 2048), (1024, 4096), (4096, 8192), (14336, 4096))
                                    for m in (8, 16, 32)
                                    for c in [affine("qmm", m, n, k, gs=32), affine("qmm_t", m, n, k, gs=32)]
                                    + [affine("splitk", m, n, k, gs=32, splits=s) for s in (2, 4, 8, 16)
                                       if k // 256 >= s]],
    # split counts 2-8 of 2-, 4- and 8-bit codes at the config-3 split shapes and three more M: a
    # count runs on 64-column tiles where those of all its partitions fit one round, else 128-column
    "route_split_tiles_bf16": [c for b in (2, 4, 8) for k, n, m in ((17408, 5120, 56), (14336, 4096, 33),
                                                                      (10752, 2048, 85), (4096, 4096, 64),
                                                                      (4096, 4096, 128), (5120, 5120, 48))
                               for c in [affine("qmm", m, n, k, bits=b)]
                               + [affine("splitk", m, n, k, bits=b, splits=s) for s in (2, 3, 4, 6, 8)]],
    "q8_0_14336x5120": [block("q8_0", 14336, 5120)],
    "q8_i8_14336x5120": [block("q8_i8", 14336, 5120)],
    "q4_k_14336x5120": [block("q4_k", 14336, 5120)],
    "blocks_14336x5120": [block("q8_0", 14336, 5120), block("q4_k", 14336, 5120)],
}
DEFAULT_WORKLOAD = "qmv_qmm_4bit_gs64_bf16"
SETTLE_S = 0.05   # seconds of untimed step replays before the timed steps


def call_name(c):
    if c["kind"] == "affine":
        head = c["route"] if c.get("B", 1) == 1 else f"{c['route']}{c['B']}"
        if c["route"] == "gather":
            head = head.replace("gather", "gathersorted" if c.get("sorted") else "gather") + f"of{c['E']}"
        if c["route"] == "splitk":
            head = f"splitk{c['splits']}"
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


def out_bytes(c):
    if c["kind"] != "affine":
        return 4 * c["N"]
    return c.get("B", 1) * c["M"] * c["N"] * (4 if c["dtype"] == F32 else 2)


def flops(c):
    return 2 * c.get("B", 1) * c["M"] * c["N"] * c["K"]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="one of: " + ", ".join(sorted(WORKLOADS)) + ", or only:<call name>")
    ap.add_argument("--calls", type=int, default=CALLS_PER_REPEAT, help="timed calls per repeat (per call, per kernel)")
    ap.add_argument("--repeats", type=int, default=REPEATS)
    ap.add_argument("--cpu-seconds", type=float, default=2.5,
                    help="target time of one single-thread oracle pass of the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--no-per-call", action="store_true", help="time whole steps only")
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
        elif c["route"] == "splitk":
            need = qmx.splitk_workspace_bytes(c["M"], c["N"], c["splits"])
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


INPUT_KEYS = ("w", "scales", "biases", "x", "blocks", "wq", "xq", "wd")


def footprint(c, d):
    return sum(d[k].numel() * d[k].element_size() for k in INPUT_KEYS if k in d)


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
    if c["route"] == "qmm_t":
        return qmx.qmm_t(d["w"], d["scales"], d["biases"], d["x"], d["out"], **kw)
    if c["route"] == "splitk":
        return qmx.qmm_t_splitk(d["w"], d["scales"], d["biases"], d["x"], d["out"], splits=c["splits"],
                                workspace=d["ws"], **kw)
    return qmx.qmm(d["w"], d["scales"], d["biases"], d["x"], d["out"], workspace=d["ws"], **kw)


def route_of(c):
    """(route name, splits) the call runs on."""
    import matmul_affine_qmv_amd as qmx
    if c["kind"] != "affine":
        return c["kind"], 1
    if c["route"] == "qmm":
        return qmx.plan(c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"])
    if c["route"] in ("batched", "gather"):
        return qmx.plan_batched(c["B"], c["M"], c["N"], c["K"], c["bits"], c["gs"], c["dtype"])
    if c["route"] == "splitk":
        return "qmm_t_splitk", c["splits"]
    return c["route"], 1


def on_matrix_cores(c, route):
    return c["kind"] == "affine" and route in ("qmm_t", "qmm_t_splitk")


# ---------------------------------------------------------------- timing
def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graphs(graphs, replays):
    """Replay graphs round-robin `replays` times; returns (wall seconds, GPU event ms)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(replays):
        graphs[k % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, start.elapsed_time(end)


def rotation_sets(c, set0, seed, dev, min_bytes=ROTATION_BYTES):
    """Set 0 plus distinct input sets until their inputs total at least
    `min_bytes`; the output (and workspace) of set 0 are shared, as one caller
    would share them."""
    n = max(2, math.ceil(min_bytes / max(1, footprint(c, set0))))
    sets = [set0]
    for r in range(1, n):
        d = make_inputs(c, seed + 104729 * r, dev)
        d["out"] = set0["out"]
        if "ws" in set0:
            d["ws"] = set0["ws"]
        sets.append(d)
    return sets


def time_per_launch(fn, sets, calls=CALLS_PER_REPEAT, repeats=REPEATS):
    """Median over `repeats` of the mean µs per launch of `fn`: a graph launches
    fn once per rotating set, replayed until at least `calls` launches are
    timed between two HIP events (after WARMUP_CALLS untimed launches)."""
    g = capture(lambda: [fn(s) for s in sets])
    n = len(sets)
    time_graphs([g], max(1, math.ceil(WARMUP_CALLS / n)))
    replays = max(1, math.ceil(calls / n))
    samples = []
    for _ in range(repeats):
        _, ms = time_graphs([g], replays)
        samples.append(1000.0 * ms / (replays * n))
    del g
    return statistics.median(samples), samples


def kernels_of(c, route, splits):
    """The kernels one call launches, each as (label, launcher over an input set,
    algorithmic bytes per launch, flops per launch, on the matrix cores).

    Algorithmic bytes are the call's own (weights, scales/biases, x, out); the
    float32 split-K partials are not counted (they are lost efficiency).  Of a
    split call, the partial kernel is credited with the inputs and the
    accumulate with the output."""
    import matmul_affine_qmv_amd as qmx
    if c["kind"] == "affine" and c["route"] in ("batched", "gather"):
        # one launch sequence for the whole batch, timed as a whole
        return [(f"qmm_{c['route']} (whole call)", lambda d, c=c: launch(c, d), alg_bytes(c), flops(c), c["M"] >= 8)]
    if c["kind"] != "affine" or route != "qmm_t_splitk":
        # the M = 1 matvecs and the block matvecs have a looped and a deep form,
        # chosen by shape inside the library: the label names both
        label = {"qmv": "qmv_kernel|qmv_deep_kernel", "qmm_t": "qmm_t_kernel",
                 "q8_0": "q8_0_kernel|q8_0_deep_kernel", "q4_k": "q4_k_kernel|q4_k_deep_kernel",
                 "q8_i8": "q8_i8_kernel"}[route if c["kind"] == "affine" else c["kind"]]
        return [(label, lambda d, c=c: launch(c, d), alg_bytes(c), flops(c), route == "qmm_t")]
    kw = dict(bits=c["bits"], group_size=c["gs"], splits=splits)
    return [
        ("qmm_t_kernel (split-K partials)",
         lambda d: qmx.qmm_t_partials(d["w"], d["scales"], d["biases"], d["x"], workspace=d["ws"], **kw),
         alg_bytes(c) - out_bytes(c), flops(c), True),
        ("splitk_accum_kernel", None, out_bytes(c), 0, False),
    ]


def partial_bytes(c, route, splits):
    """float32 split-K partial traffic of one call (written once, read once)."""
    if route != "qmm_t_splitk":
        return 0
    return 2 * splits * c.get("B", 1) * c["M"] * c["N"] * 4


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


# ---------------------------------------------------------------- calibration
def calibrate(dev, sizes, calls, repeats):
    """Achievable rates on this GPU: a streaming read of 512 MiB (and of each
    size in `sizes`, rotating over at least 512 MiB), a streaming copy of
    512 MiB, back-to-back bf16 MFMAs on every SIMD, and an empty launch."""
    import torch

    from matmul_affine_qmv_amd import calib
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    big = [torch.empty(ROTATION_BYTES // 4, dtype=torch.int32, device=dev).random_() for _ in range(2)]
    grids = (4 * cus, 8 * cus, 16 * cus, 64 * cus)   # the fastest grid of these counts
    us = min(time_per_launch(lambda t, b=b: calib.read(t, sink, b), big, calls=20, repeats=repeats)[0] for b in grids)
    res = {"read_gbs_512mib": ROTATION_BYTES / us / 1e3}
    dst = torch.empty_like(big[0])
    us = min(time_per_launch(lambda t, b=b: calib.copy(t, dst, b), big, calls=20, repeats=repeats)[0] for b in grids)
    res["copy_gbs_512mib"] = 2 * ROTATION_BYTES / us / 1e3
    del dst, big
    at = {}
    for name, nbytes in sizes.items():
        nbytes = max(16, nbytes // 16 * 16)
        n = max(2, math.ceil(ROTATION_BYTES / nbytes))
        bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(n)]
        us = min(time_per_launch(lambda t, b=b: calib.read(t, sink, b), bufs, calls=calls, repeats=repeats)[0]
                 for b in grids[:3])
        at[name] = {"bytes": nbytes, "us": us, "gbs": nbytes / us / 1e3}
        del bufs
    res["read_at_call_size"] = at
    out = torch.empty(16 * cus * 256, dtype=torch.float32, device=dev)
    iters = 200
    for shape in (32, 16):
        us, _ = time_per_launch(lambda _, s=shape: calib.mfma(out, iters, 16 * cus, s), [None, None], calls=10,
                                repeats=repeats)
        res[f"mfma_bf16_tflops_{shape}x{shape}"] = calib.mfma_flops(iters, 16 * cus) / us / 1e6
    # Matrix-core / vector-ALU co-issue, two waves per SIMD: cycles per SIMD (at
    # the 2.4 GHz peak clock) for one 32x32x16 MFMA followed by F float FMAs,
    # against the MFMA alone and the FMAs alone.
    co, co_iters = {}, 1000
    for f in calib.MFMA_VALU_FMAS:
        row = {}
        for with_mfma in (True, False):
            if f == 0 and not with_mfma:
                continue
            us, _ = time_per_launch(lambda _, f=f, w=with_mfma: calib.mfma_valu(out, co_iters, 2 * cus, f, w),
                                    [None, None], calls=10, repeats=repeats)
            # 2*cus work-groups of 4 waves: two waves per SIMD, 4 rounds per iteration
            row["mfma_plus_fma" if with_mfma else "fma_only"] = round(us * 1e-6 * 2.4e9 / (co_iters * 4 * 2), 1)
        co[f"fma_per_mfma_{f}"] = row
    res["mfma_valu_cycles_per_simd_round"] = co
    us, _ = time_per_launch(lambda _: calib.empty(1), [None] * 100, calls=1000, repeats=repeats)
    res["empty_launch_us"] = us
    return res


# ---------------------------------------------------------------- oracle baseline
def cpu_model():
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.strip().startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(calls, set0, target_1t_s, repeats=REPEATS):
    """The float64 oracle on an evenly spaced sample of output columns of every
    call (input set 0): median of `repeats` passes on 1 thread and on every host
    core; the GPU outputs of the sampled columns are checked against it."""
    import numpy as np

    import matmul_affine_qmv_amd as qmx
    import oracle
    import qmx_inputs as qi
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare

    orc = oracle.load()
    host = []
    for i, c in enumerate(calls):
        d = set0[i]
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

    def one_call(i, c, cols):
        h = host[i]
        if c["kind"] == "affine":
            return orc.affine(h["w"], h["scales"], h["biases"], c["dtype"], h["x"], c["dtype"], c["M"], c["N"],
                              c["K"], c["bits"], c["gs"], cols=cols)
        if c["kind"] == "q8_0":
            return orc.q8_0(h["blocks"], h["x"], c["N"], c["K"], rows=cols)
        if c["kind"] == "q8_i8":
            return orc.q8_i8(h["wq"], h["xq"], h["wd"], c["N"], c["K"], rows=cols)
        return orc.q4_k(h["blocks"], h["x"], c["N"], c["K"], rows=cols)

    def columns(c, frac):
        n = max(8, int(round(c["N"] * frac)))
        return np.linspace(0, c["N"] - 1, num=min(n, c["N"]), dtype=np.int64).astype(np.int32)

    cores = host_cores()
    # single-thread rate on a small slice of the first call sizes the sample
    orc.set_num_threads(1)
    probe = columns(calls[0], 0.01)
    t0 = time.perf_counter()
    one_call(0, calls[0], probe)
    rate = calls[0]["M"] * len(probe) * calls[0]["K"] / max(time.perf_counter() - t0, 1e-6)   # MACs/s
    macs = sum(c["M"] * c["N"] * c["K"] for c in calls)   # the oracle takes one problem of a batch
    frac = min(1.0, target_1t_s * rate / max(1, macs))
    cols = [columns(c, frac) for c in calls]
    sample_bytes = sum(alg_bytes(dict(c, B=1, E=1, route="qmm")) * len(cl) / c["N"] for c, cl in zip(calls, cols))

    def timed_pass(threads):
        orc.set_num_threads(threads)
        t0 = time.perf_counter()
        refs = [one_call(i, c, cl) for i, (c, cl) in enumerate(zip(calls, cols))]
        return time.perf_counter() - t0, refs

    t1 = [timed_pass(1)[0] for _ in range(repeats)]
    tn, refs = [], None
    for _ in range(repeats):
        t, refs = timed_pass(cores)
        tn.append(t)
    worst = None
    for c, cl, ref, h in zip(calls, cols, refs, host):
        got = qi.storage_to_f64(h["out"], c["dtype"])
        got = got[:, cl] if got.ndim == 2 else got[cl]
        m = compare(got, ref, c["dtype"], orc)
        score = m["rel_l2"] / m["rel_gate"]
        if worst is None or not m["ok"] or (worst[2] and score > worst[1]):
            worst = (call_name(c), score, m["ok"])
    med1, medn = statistics.median(t1), statistics.median(tn)
    return {
        "value": sample_bytes / medn / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"float64 C oracle on an evenly spaced {100 * frac:.2f}% of the output columns of every call "
                   f"(input set 0, {sample_bytes / 1e6:.1f} MB of algorithmic bytes); median of {repeats} passes "
                   f"on {cores} threads ({medn:.2f} s) and on 1 thread ({med1:.2f} s)"),
        "single_thread": {"value": sample_bytes / med1 / 1e9, "unit": "GB/s", "cores": 1, "median_s": med1,
                          "runs_s": t1},
        "all_cores": {"median_s": medn, "runs_s": tn},
        "nproc": cores,
        "cpu_model": cpu_model(),
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
    say = lambda *a: print("bench:", *a, file=sys.stderr, flush=True)   # noqa: E731

    # whole-step input sets: at least 3x the MALL is touched between two uses of a set
    set0 = [make_inputs(c, args.seed + 7919 * i, dev) for i, c in enumerate(calls)]
    per_set = sum(footprint(c, d) for c, d in zip(calls, set0))
    nsets = max(3, math.ceil(3 * MALL_BYTES / per_set))
    sets = [set0] + [[make_inputs(c, args.seed + 104729 * r + 7919 * i, dev) for i, c in enumerate(calls)]
                     for r in range(1, nsets)]
    # the split-K partials of every call and set go to one scratch workspace, as a
    # runtime's scratch arena would hold them (the per-call rotations below share
    # set 0's the same way); the calls run in order on one stream
    ws_need = max((d["ws"].numel() for s in sets for d in s if d.get("ws") is not None), default=0)
    if ws_need:
        scratch = torch.empty(ws_need, dtype=torch.float32, device=dev)
        for s in sets:
            for d in s:
                if d.get("ws") is not None:
                    d["ws"] = scratch[: d["ws"].numel()]
    torch.cuda.synchronize()

    # eager warm-up (loads code objects, caches the CU count), then capture one graph per set
    for s in sets:
        for c, d in zip(calls, s):
            launch(c, d)
    torch.cuda.synchronize()
    graphs = [capture(lambda s=s: [launch(c, d) for c, d in zip(calls, s)]) for s in sets]
    warm = max(args.warmup, 1) * len(graphs)
    t_warm, _ = time_graphs(graphs, warm)
    # more untimed replays until the GPU has been busy for SETTLE_S, so that its
    # clock has ramped up before the timed steps (50 steps of the default
    # workload measured 3-5% slower per step than 200 without this)
    extra = math.ceil(max(0.0, SETTLE_S - t_warm) / (t_warm / warm))
    if extra:
        time_graphs(graphs, extra)
    say(f"{len(calls)} calls, {nsets} step sets of {per_set / 1e6:.1f} MB; timing {args.steps} steps")
    wall, gpu_ms = time_graphs(graphs, args.steps)
    step_bytes = sum(alg_bytes(c) for c in calls)
    step_flops = sum(flops(c) for c in calls)
    value = args.steps * step_bytes / wall / 1e9
    del graphs
    sets = sets[:1]   # free the other step sets; set 0 seeds the per-call rotations

    details, kernels = [], []
    if not args.no_per_call:
        for i, c in enumerate(calls):
            route, splits = route_of(c)
            rot = rotation_sets(c, set0[i], args.seed + 7919 * i, dev)
            us, samples = time_per_launch(lambda d, c=c: launch(c, d), rot, args.calls, args.repeats)
            shown = route if route != "qmm_t_splitk" else f"qmm_t_splitk{splits}"
            det = {"call": call_name(c), "route": shown, "us": us, "us_repeats": samples, "rotating_sets": len(rot),
                   "rotation_bytes": footprint(c, set0[i]) * len(rot), "alg_bytes": alg_bytes(c),
                   "gbs": alg_bytes(c) / us / 1e3, "hbm_frac": alg_bytes(c) / us / 1e3 / HBM_PEAK_GBS,
                   "tflops": flops(c) / us / 1e6, "partial_bytes": partial_bytes(c, route, splits),
                   "roofline": roofline_for(c, us, matrix=on_matrix_cores(c, route))}
            if on_matrix_cores(c, route):
                det["mfma_frac"] = flops(c) / us / 1e6 / MFMA_BF16_TFLOPS
            details.append(det)
            for label, fn, kb, kf, matrix in kernels_of(c, route, splits):
                if fn is None:   # the accumulate: the call's time less the partial kernel's
                    kus = us - kernels[-1]["us"]
                    how = "call time less the partial kernel's"
                else:
                    kus, _ = time_per_launch(fn, rot, args.calls, args.repeats)
                    how = "measured"
                kernels.append({"call": call_name(c), "kernel": label, "us": kus, "how": how, "alg_bytes": kb,
                                "flops": kf, "roofline": roofline_for(c, kus, kb, kf, matrix)})
            say(f"{call_name(c)}: {shown} {us:.2f} us ({det['hbm_frac']:.3f} of HBM), {len(rot)} sets")
            del rot
            torch.cuda.empty_cache()

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
    }
    if details:
        dom = max(kernels, key=lambda k: k["us"])
        dcall = next(d for d in details if d["call"] == dom["call"])
        roof = dict(dom["roofline"])
        traffic, traffic_src = stored_traffic(dom["call"], dom["kernel"])
        roof.update({"traffic": traffic, "kernel": dom["kernel"], "call": dom["call"], "us_per_launch": dom["us"],
                     "alg_bytes_per_launch": dom["alg_bytes"], "flops_per_launch": dom["flops"],
                     "traffic_source": traffic_src, "call_us": dcall["us"],
                     "call_frac": dcall["roofline"]["frac"], "call_bound": dcall["roofline"]["bound"],
                     "partial_bytes_per_call_excluded": dcall["partial_bytes"]})
        line.update({
            "us_per_call": {d["call"]: round(d["us"], 3) for d in details},
            "gbs_per_call": {d["call"]: round(d["gbs"], 1) for d in details},
            "hbm_frac_per_call": {d["call"]: round(d["hbm_frac"], 4) for d in details},
            "tflops_per_call": {d["call"]: round(d["tflops"], 2) for d in details if "mfma_frac" in d},
            "mfma_frac_per_call": {d["call"]: round(d["mfma_frac"], 4) for d in details if "mfma_frac" in d},
            "roofline_frac_per_call": {d["call"]: round(d["roofline"]["frac"], 4) for d in details},
            "routes": {d["call"]: d["route"] for d in details},
            "us_per_kernel": {f"{k['call']}:{k['kernel']}": round(k["us"], 3) for k in kernels},
            "roofline": roof,
            "protocol": {"rotation_min_bytes": ROTATION_BYTES, "calls_per_repeat_min": args.calls,
                         "repeats": args.repeats, "statistic": "median", "warmup_calls": WARMUP_CALLS},
        })
    if not args.no_calibration and details:
        say("calibration")
        cal = calibrate(dev, {d["call"]: d["alg_bytes"] for d in details}, args.calls, args.repeats)
        line["achievable"] = cal
        rd = line["roofline"]
        at = cal["read_at_call_size"].get(rd["call"])
        if at:
            rd["achievable_read_us_at_call_bytes"] = at["us"]
            rd["call_frac_of_achievable_read"] = at["us"] / rd["call_us"]
    if not args.no_cpu_baseline:
        say("cpu baseline")
        # the rotations share set 0's outputs: compute set 0's once more before checking them
        for c, d in zip(calls, set0):
            launch(c, d)
        torch.cuda.synchronize()
        line["cpu_baseline"] = cpu_baseline(calls, set0, args.cpu_seconds, args.repeats)
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump({"line": line, "details": details, "kernels": kernels}, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
