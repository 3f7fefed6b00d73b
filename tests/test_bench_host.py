"""Host logic of bench.py (no GPU): byte and flop accounting, the roofline
choice, workload resolution and the one-GPU rule.

The expected byte counts are the figures stated for these workloads as the
bytes a call must move once, N*K*b/8 + 2*N*(K/gs)*|S| + M*K*|X| + M*N*|O|
(plus the block formats' own sizes), written out here as numbers rather than
recomputed from that formula.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

F32, F16, BF16 = bench.F32, bench.F16, bench.BF16


@pytest.mark.parametrize("c,expected", [
    # matvec, 4096 x 4096 4-bit gs 64, float32 everywhere
    (bench.affine("qmv", 1, 4096, 4096, dt=F32), 10_518_528),
    # the small-M matmul shapes in bfloat16, (K, N, M)
    (bench.affine("qmm", 22, 2048, 2048), 2_539_520),
    (bench.affine("qmm", 16, 4096, 4096), 9_699_328),
    (bench.affine("qmm", 16, 4096, 256), 729_088),
    (bench.affine("qmm", 85, 2048, 10752), 14_562_304),
    (bench.affine("qmm", 33, 4096, 14336), 34_246_656),
    (bench.affine("qmm", 56, 5120, 17408), 52_658_176),
    # block formats, 14336 x 5120, float32 x and out
    (bench.block("q8_0", 14336, 5120), 82_653_184),
    (bench.block("q4_k", 14336, 5120), 41_365_504),
])
def test_alg_bytes_match_stated_figures(c, expected):
    assert bench.alg_bytes(c) == expected


def test_alg_bytes_16bit_matvec_shapes():
    # 16-bit x, scales, biases and out: 14.8 / 41.3 / 41.3 / 79.7 MB
    got = [bench.alg_bytes(bench.affine("qmv", 1, n, k)) / 1e6 for n, k in bench.QMV_SHAPES]
    assert [round(g, 1) for g in got] == [14.8, 41.3, 41.3, 79.7]


def test_batched_and_gather_bytes():
    one = bench.alg_bytes(bench.affine("qmm", 16, 2048, 4096))
    assert bench.alg_bytes(bench.affine("batched", 16, 2048, 4096, B=8)) == 8 * one
    # a gather counts each of its E weight matrices once, x and out once per problem
    w = 2048 * 4096 // 2 + 2 * 2048 * 64 * 2
    xo = 4096 * 2 + 2048 * 2
    g = bench.affine("gather", 1, 2048, 4096, B=16, E=8)
    assert bench.alg_bytes(g) == 8 * w + 16 * xo
    assert bench.alg_bytes(bench.affine("gather", 1, 2048, 4096, B=16, E=8, sorted_idx=True)) == bench.alg_bytes(g)


def test_split_kernels_bytes():
    """Algorithmic bytes of a split call are the call's own: the partial kernel
    is credited with the inputs, the accumulate with the 16-bit output, and the
    S*M*N float32 partials count for neither (they show up as lost efficiency
    and are reported on their own)."""
    c = bench.affine("qmm", 56, 5120, 17408)
    (lp, fnp, bp, fp, mp), (la, fna, ba, fa, ma) = bench.kernels_of(c, "qmm_t_splitk", 6)
    assert bp == 52_658_176 - 56 * 5120 * 2 == 52_084_736
    assert ba == 56 * 5120 * 2
    assert bp + ba == bench.alg_bytes(c)
    assert fp == 2 * 56 * 5120 * 17408 and fa == 0 and mp and not ma
    assert fnp is not None and fna is None   # the accumulate is the call's time less the partial kernel's
    assert bench.partial_bytes(c, "qmm_t_splitk", 6) == 2 * 6 * 56 * 5120 * 4
    assert bench.partial_bytes(c, "qmm_t", 1) == 0


def test_forced_split_workload_keeps_256_columns_per_partition():
    calls = bench.WORKLOADS["qmm_splits_4bit_gs64_bf16"]
    for c in calls:
        if c["route"] == "splitk":
            assert c["splits"] in (2, 3, 4) and c["K"] >= 512 and c["K"] // c["splits"] >= 256
    got = {(c["K"], c["splits"]) for c in calls if c["route"] == "splitk"}
    assert (256, 2) not in got and (17408, 4) in got and (2048, 3) in got
    # every shape also runs unsplit
    assert len([c for c in calls if c["route"] == "qmm_t"]) == len(bench.QMM_SHAPES)


def test_sweep_workload_covers_the_grid():
    calls = bench.WORKLOADS["sweep_4096"]
    assert len(calls) == 3 * 3 * 2 * 5
    assert {(c["bits"], c["gs"], c["dtype"], c["M"]) for c in calls} == {
        (b, g, d, m) for b in (2, 4, 8) for g in (32, 64, 128) for d in (F16, BF16) for m in (1, 8, 33, 128, 257)}


def test_roofline_bound_choice():
    # M = 56: HBM time (6.58 us) above MFMA time (4.0 us) at the published peaks
    r = bench.roofline_for(bench.affine("qmm", 56, 5120, 17408), 32.0)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(52_658_176 / 32e-6 / 1e9)
    assert r["frac"] == pytest.approx(r["achieved"] / 8000.0)
    # M = 512 on 4096 x 4096: 17.2 GFLOP outweighs 17.8 MB
    r = bench.roofline_for(bench.affine("qmm", 512, 4096, 4096), 40.0)
    assert r["bound"] == "mfma" and r["peak"] == 2500.0
    assert r["achieved"] == pytest.approx(2 * 512 * 4096 * 4096 / 40e-6 / 1e12)
    # the vector route is never priced on the matrix cores
    assert bench.roofline_for(bench.affine("qmv", 1, 4096, 4096), 5.0)["bound"] == "hbm"


def test_workloads_resolve_with_unique_call_names():
    for name, calls in bench.WORKLOADS.items():
        names = [bench.call_name(c) for c in calls]
        assert len(set(names)) == len(names), name
        assert bench.resolve_workload(name) is calls
        for n in names:
            assert [bench.call_name(c) for c in bench.resolve_workload("only:" + n)] == [n]
    assert len(bench.WORKLOADS[bench.DEFAULT_WORKLOAD]) == 10
    with pytest.raises(SystemExit):
        bench.resolve_workload("no_such_workload")
    with pytest.raises(SystemExit):
        bench.resolve_workload("only:no_such_call")


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
