"""HIP path against the float64 oracle, through the C ABI (needs a gfx950 GPU).

Small cases cover several tiles and ragged tails and are checked on every
output; the full workload sizes are checked on sampled columns (all rows)
that the oracle computes one by one.  Every case prints its name before it
touches the GPU.
"""
import sys

import numpy as np
import pytest

import qmx_inputs as qi
from parity import assert_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import matmul_affine_qmv_amd as qmx  # noqa: E402

DEV = "cuda:0"
ALL_BITS = [1, 2, 3, 4, 5, 6, 8]
ODD_BITS = [1, 3, 5, 6]          # widths whose fields may straddle words (1 bit: 32 codes per word)
TORCH_DT = {qi.F32: torch.float32, qi.F16: torch.float16, qi.BF16: torch.bfloat16}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_dev(case):
    dt = case["dtype"]
    return (qmx.words_tensor(case["w"], DEV), qmx.storage_tensor(case["scales"], dt, DEV),
            qmx.storage_tensor(case["biases"], dt, DEV), qmx.storage_tensor(case["x"], dt, DEV))


def out64(t, dt):
    return qi.storage_to_f64(qmx.tensor_bits(t), dt)


def sample_cols(N, count, seed):
    if N <= count:
        return np.arange(N, dtype=np.int32)
    rng = np.random.Generator(np.random.PCG64(seed))
    edge = np.r_[0:16, N - 16:N]
    rest = rng.choice(np.arange(16, N - 16), size=count - edge.size, replace=False)
    return np.unique(np.r_[edge, rest]).astype(np.int32)


def run(route, w, s, b, x, bits, gs, splits=None, workspace=None):
    if route == "qmv":
        return qmx.qmv(w, s, b, x, bits=bits, group_size=gs)
    if route == "qmm_t":
        return qmx.qmm_t(w, s, b, x, bits=bits, group_size=gs)
    if route == "splitk":
        return qmx.qmm_t_splitk(w, s, b, x, bits=bits, group_size=gs, splits=splits, workspace=workspace)
    return qmx.qmm(w, s, b, x, bits=bits, group_size=gs)


def check_affine(orc, route, M, N, K, bits, gs, dt, seed, splits=None, cols=None, bias="jitter",
                 reruns=0):
    say(route, f"M={M} N={N} K={K} bits={bits} gs={gs} dt={qi.DTYPE_NAMES[dt]} splits={splits} seed={seed}")
    c = qi.affine_case(M, N, K, bits, gs, dt, seed=seed, bias=bias)
    w, s, b, x = to_dev(c)
    y = run(route, w, s, b, x, bits, gs, splits)
    torch.cuda.synchronize()
    got = out64(y, dt)
    ref = orc.affine_case(c, cols=cols)
    if cols is not None:
        got = got[:, cols]
    m = assert_close(got, ref, dt, orc, what=f"{route} {M}x{N}x{K} b{bits} gs{gs} dt{dt} S{splits}")
    for _ in range(reruns):
        y2 = run(route, w, s, b, x, bits, gs, splits)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32),
                           y2.view(torch.int16) if y2.dtype != torch.float32 else y2.view(torch.int32)), \
            "rerun not bit-identical"
    return m


# ---------------------------------------------------------------- qmv
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [qi.F32, qi.F16, qi.BF16])
def test_qmv_small_all_formats(orc, bits, gs, dt):
    # ragged N (not a multiple of 4 rows), K spanning several 64-lane chunk rounds plus a tail
    K = 2560 if bits != 2 else 2560
    check_affine(orc, "qmv", 1, 67, K, bits, gs, dt, seed=1000 + bits * 100 + gs + dt)


@pytest.mark.parametrize("M", [2, 3, 5, 7])
def test_qmv_small_m(orc, M):
    check_affine(orc, "qmv", M, 45, 1024, 4, 64, qi.BF16, seed=1100 + M)
    check_affine(orc, "qmv", M, 18, 512, 8, 32, qi.F32, seed=1150 + M)
    for bits in ODD_BITS:
        check_affine(orc, "qmv", M, 29, 640, bits, 32 if bits != 6 else 128, qi.F16 if bits < 4 else qi.BF16,
                     seed=1170 + 10 * M + bits)
        check_affine(orc, "qmv", M, 13, 384, bits, 64, qi.F32, seed=1190 + 10 * M + bits)


@pytest.mark.parametrize("N,K,bits,dt", [(67, 256, 4, qi.BF16), (8192, 256, 4, qi.F16), (16384, 256, 4, qi.BF16),
                                          (67, 1536, 8, qi.F32), (67, 2560, 8, qi.BF16), (2048, 2560, 8, qi.F16),
                                          (6000, 2560, 4, qi.BF16)])
def test_qmv_work_splits(orc, N, K, bits, dt):
    """Shapes for which the M = 1 split rule picks each of its work splits (waves
    per row tile x row groups per wave: 1x1, 1x2, 1x4, 2x1, 4x1, 5x2, 5x4);
    ragged N where the shape allows."""
    check_affine(orc, "qmv", 1, N + (3 if N > 4000 else 0), K, bits, 64, dt, seed=1160 + N + K + bits)


@pytest.mark.parametrize("N,K", [(67, 2048), (4093, 992), (1000, 1056), (2045, 4096), (4096, 2080), (3001, 4064),
                                 (4097, 4096), (2048, 4128), (2029, 4096), (8195, 4160), (4100, 6144), (8192, 6176)])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [qi.F32, qi.F16, qi.BF16])
def test_qmv_deep_rounds(orc, N, K, gs, dt):
    """M = 1 rows of 4-bit codes short enough for all rounds of 64 chunks per wave
    in flight (on a 256-CU part, 16-bit x: up to 256 work-groups of 16 rows,
    two rounds from 128 work-groups; float32 x: two or three rounds with 4 rows
    per wave from N = 8192, 2 rows from N = 4096): ragged last rounds and ragged
    N, and the neighbours just past each limit (one work-group too many or too
    few, K one chunk too long), which take the looped kernel."""
    if K % gs:
        pytest.skip("K is not a multiple of the group size")
    check_affine(orc, "qmv", 1, N, K, 4, gs, dt, seed=1300 + N + K + gs + dt)


@pytest.mark.parametrize("bits", ODD_BITS)
@pytest.mark.parametrize("N,K", [(67, 256), (16384, 256), (67, 1536), (2048, 2560), (6000, 5120), (21, 14336)])
def test_qmv_odd_width_work_splits(orc, bits, N, K):
    """The 32-code chunks of the odd widths under every kind of work split the
    M = 1 rule picks for them, including long rows split over several waves."""
    check_affine(orc, "qmv", 1, N + (3 if N > 4000 else 0), K, bits, 64, qi.BF16 if bits != 5 else qi.F16,
                 seed=1400 + N + K + bits)


def test_qmv_config1_full(orc):
    # M=1, N=K=4096, 4-bit gs64, float32 everywhere (all outputs checked, reruns bit-identical)
    check_affine(orc, "qmv", 1, 4096, 4096, 4, 64, qi.F32, seed=qi.seed_for(1, 0), reruns=2)


@pytest.mark.parametrize("NK", [(5120, 5120), (14336, 5120), (5120, 14336), (27648, 5120)])
@pytest.mark.parametrize("dt", [qi.F32, qi.F16, qi.BF16])
def test_qmv_config2_full(orc, NK, dt):
    N, K = NK
    check_affine(orc, "qmv", 1, N, K, 4, 64, dt, seed=qi.seed_for(2, N // 1024 + K // 1024 + dt))


# ---------------------------------------------------------------- qmm_t and split-K
@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8, 9, 16, 22, 33, 56, 85, 128, 129, 200])
def test_qmm_t_small_m_tails(orc, M):
    check_affine(orc, "qmm_t", M, 200, 512, 4, 64, qi.BF16, seed=1200 + M)


@pytest.mark.parametrize("M,N,K", [(3, 14336, 5120), (7, 27648, 5120), (5, 5120, 5120), (3, 8192, 4096)])
def test_small_m_matrix_route(orc, M, N, K):
    """M < 8 shapes that the policy sends to the matrix cores (sampled columns)."""
    assert qmx.plan(M, N, K, 4, 64, qi.BF16)[0] != "qmv"
    check_affine(orc, "qmm", M, N, K, 4, 64, qi.BF16, seed=1250 + M, cols=sample_cols(N, 256, M), reruns=1)


# (M, N, K): 2/4/8-bit unsplit qmm_t with M <= 32 and few 128-column tiles runs on
# 32-column tiles whose 8 waves split each 512-column K block: 16- and 32-row
# tiles, ragged N, one to five blocks, K ranges whose scales and biases are
# staged whole or per block (K / group size not a multiple of 8).
NARROW_SHAPES = [(16, 1000, 1536), (32, 96, 2560), (9, 33, 512), (25, 4100, 1024), (1, 70, 1024)]


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [qi.F16, qi.BF16])
def test_qmm_t_narrow_tiles(orc, bits, gs, dt):
    for i, (M, N, K) in enumerate(NARROW_SHAPES):
        check_affine(orc, "qmm_t", M, N, K, bits, gs, dt, seed=1280 + 10 * i + bits + gs + dt, reruns=1)


def test_qmm_narrow_policy_shapes(orc):
    """The shapes the policy sends unsplit to 32-column tiles (they would split K
    on 128-column tiles): the config-3 M = 22 and M = 16 calls, M = 8 of the
    4096 x 4096 sweep at 2, 4 and 8 bits, and 14336 x 4096, whose 448 tiles take
    two rounds of the chip, every output against the oracle."""
    for M, N, K, bits in ((22, 2048, 2048, 4), (16, 4096, 4096, 4), (8, 4096, 4096, 4), (8, 4096, 4096, 8),
                          (8, 4096, 4096, 2), (16, 14336, 4096, 4)):
        assert qmx.plan(M, N, K, bits, 64, qi.BF16, num_cus=256) == ("qmm_t", 1)
        check_affine(orc, "qmm", M, N, K, bits, 64, qi.BF16, seed=1290 + M + bits, reruns=1)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [qi.F16, qi.BF16])
def test_qmm_t_small_all_formats(orc, bits, gs, dt):
    check_affine(orc, "qmm_t", 37, 160, 768, bits, gs, dt, seed=1300 + bits * 100 + gs + dt)
    check_affine(orc, "splitk", 37, 160, 768, bits, gs, dt, seed=1300 + bits * 100 + gs + dt, splits=3)


@pytest.mark.parametrize("splits", [2, 3, 4, 5, 8])
def test_splitk_every_count(orc, splits):
    check_affine(orc, "splitk", 22, 384, 2048, 4, 64, qi.BF16, seed=1400 + splits, splits=splits, reruns=2)


CONFIG3 = [(2048, 2048, 22), (4096, 4096, 16), (256, 4096, 16), (10752, 2048, 85), (14336, 4096, 33),
           (17408, 5120, 56), (4096, 4096, 512)]


@pytest.mark.parametrize("KNM", CONFIG3)
def test_qmm_config3_policy(orc, KNM):
    K, N, M = KNM
    cols = sample_cols(N, 384, seed=K + N + M)
    check_affine(orc, "qmm", M, N, K, 4, 64, qi.BF16, seed=qi.seed_for(3, M), cols=cols, reruns=1)


@pytest.mark.parametrize("KNM", [(2048, 2048, 22), (4096, 4096, 16), (10752, 2048, 85), (14336, 4096, 33),
                                 (17408, 5120, 56)])
@pytest.mark.parametrize("route", ["qmm_t", "s2", "s3", "s4"])
def test_qmm_config3_every_route(orc, KNM, route):
    K, N, M = KNM
    cols = sample_cols(N, 256, seed=K + N + M + 1)
    if route == "qmm_t":
        check_affine(orc, "qmm_t", M, N, K, 4, 64, qi.BF16, seed=qi.seed_for(3, M), cols=cols)
    else:
        check_affine(orc, "splitk", M, N, K, 4, 64, qi.BF16, seed=qi.seed_for(3, M), cols=cols,
                     splits=int(route[1:]))


def partition_groups(K, S, p, gs):
    """Groups [g0, g1) of split-K partition p: K in segments of 256 columns (128
    when K is not a multiple of 256), partition p taking segments
    [floor(p*nseg/S), floor((p+1)*nseg/S))."""
    seg = 256 if K % 256 == 0 else 128
    nseg = K // seg
    return (p * nseg // S) * seg // gs, ((p + 1) * nseg // S) * seg // gs


# (M, N, K, S): 64-column tiles (tiles x S within one round of a 256-CU part),
# 128-column tiles (N = 8192: beyond it), and K not a multiple of 256
@pytest.mark.parametrize("M,N,K,S", [(22, 256, 1792, 3), (56, 256, 4352, 5), (22, 8192, 1792, 3), (22, 256, 1152, 3),
                                     (85, 320, 2560, 4)])
def test_splitk_partials_match_partition_oracle(orc, M, N, K, S):
    """workspace[p] is the float32 partial of partition p over its segments of
    K, on either tile width."""
    bits, gs, dt = 4, 64, qi.BF16
    say("splitk partials", M, N, K, S)
    c = qi.affine_case(M, N, K, bits, gs, dt, seed=1500)
    w, s, b, x = to_dev(c)
    ws = torch.empty(S * M * N, dtype=torch.float32, device=DEV)
    y = qmx.qmm_t_splitk(w, s, b, x, bits=bits, group_size=gs, splits=S, workspace=ws)
    torch.cuda.synchronize()
    parts = ws.view(S, M, N).cpu().numpy().astype(np.float64)
    for p in range(S):
        g0, g1 = partition_groups(K, S, p, gs)
        ref = orc.affine_groups(c["w"], c["scales"], c["biases"], dt, c["x"], dt, M, N, K, bits, gs, g0, g1)
        assert_close(parts[p], ref, qi.F32, orc, what=f"partial {p}")
    # the output is the rounded sum of the partials in ascending order
    acc = parts[0].astype(np.float32)
    for p in range(1, S):
        acc = (acc + parts[p].astype(np.float32)).astype(np.float32)
    want = orc.round(acc.astype(np.float64), dt)
    assert np.array_equal(out64(y, dt), want)


@pytest.mark.parametrize("bits,gs,dt", [(4, 64, qi.BF16), (2, 32, qi.F16), (8, 128, qi.BF16)])
def test_partials_and_accumulate_entry_points(orc, bits, gs, dt):
    """qmx_qmm_t_partials writes exactly the partition partials qmx_qmm_t_splitk
    leaves in its workspace, and qmx_splitk_accumulate of those partials gives
    qmx_qmm_t_splitk's output bit for bit; the workspace's contents on entry
    (random bytes here, then the first call's) do not matter."""
    M, N, K, S = 33, 384, 2560, 4
    say("partials + accumulate", M, N, K, bits, gs, dt, S)
    c = qi.affine_case(M, N, K, bits, gs, dt, seed=1600 + bits + gs)
    w, s, b, x = to_dev(c)
    g = torch.Generator(device="cpu").manual_seed(1650 + bits + gs)
    words = qmx.splitk_workspace_bytes(M, N, S) // 4
    ws_a = torch.randint(-2**31, 2**31 - 1, (words,), generator=g, dtype=torch.int32).to(DEV).view(torch.float32)
    y = qmx.qmm_t_splitk(w, s, b, x, bits=bits, group_size=gs, splits=S, workspace=ws_a)
    y2 = qmx.qmm_t_splitk(w, s, b, x, bits=bits, group_size=gs, splits=S, workspace=ws_a)
    parts = qmx.qmm_t_partials(w, s, b, x, bits=bits, group_size=gs, splits=S)
    out = torch.empty_like(y)
    qmx.splitk_accumulate(parts, out, S)
    torch.cuda.synchronize()
    assert torch.equal(parts.reshape(-1).view(torch.int32), ws_a.view(torch.int32))
    assert torch.equal(out.view(torch.int16), y.view(torch.int16))
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    host = parts.cpu().numpy().astype(np.float64)
    for p in range(S):
        g0, g1 = partition_groups(K, S, p, gs)
        ref = orc.affine_groups(c["w"], c["scales"], c["biases"], dt, c["x"], dt, M, N, K, bits, gs, g0, g1)
        assert_close(host[p], ref, qi.F32, orc, what=f"partial {p}")


def test_accumulate_sums_in_order_and_rounds_once(orc):
    """The accumulate kernel alone on float32 partials chosen so that the
    summation order and a single rounding are visible: ascending float32 sums
    of the partitions, then one round-to-nearest-even to the output type."""
    M, N = 7, 130   # M*N not a multiple of 4: the element-wise tail path too
    rng = np.random.Generator(np.random.PCG64(77))
    for S in (2, 3, 16):
        for dt in (qi.BF16, qi.F16):
            say("accumulate", M, N, S, dt)
            parts = (rng.standard_normal((S, M, N)) * rng.choice([1e-3, 1.0, 1e3], size=(S, M, N))).astype(np.float32)
            ws = torch.from_numpy(parts.reshape(-1)).to(DEV)
            out = torch.empty((M, N), dtype=TORCH_DT[dt], device=DEV)
            qmx.splitk_accumulate(ws, out, S)
            torch.cuda.synchronize()
            acc = parts[0].copy()
            for p in range(1, S):
                acc = (acc + parts[p]).astype(np.float32)
            want = orc.round(acc.astype(np.float64), dt)
            assert np.array_equal(out64(out, dt), want)


@pytest.mark.parametrize("bits,gs,dt", [(4, 64, qi.BF16), (2, 32, qi.F16), (8, 128, qi.F16), (2, 128, qi.BF16),
                                        (3, 64, qi.BF16), (5, 32, qi.F16), (6, 128, qi.BF16), (1, 64, qi.F16)])
def test_scale_bias_alignment_paths(orc, bits, gs, dt):
    """Scales/biases that start 2 bytes past a 16-byte boundary cannot be staged in
    16-byte chunks; the per-block path must give the same bits as the staged one."""
    M, N, K, S = 40, 256, 4096, 4
    say("scale/bias alignment", M, N, K, bits, gs, dt, S)
    c = qi.affine_case(M, N, K, bits, gs, dt, seed=1700 + bits + gs)
    w, s, b, x = to_dev(c)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    s2, b2 = shifted(s), shifted(b)
    assert s2.data_ptr() % 16 != 0
    for route, kw in (("qmm_t", {}), ("splitk", {"splits": S})):
        y_a = run(route, w, s, b, x, bits, gs, **kw)
        y_b = run(route, w, s2, b2, x, bits, gs, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y_a.view(torch.int16), y_b.view(torch.int16)), route
        assert_close(out64(y_b, dt), orc.affine_case(c), dt, orc, what=f"{route} shifted scales")


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_splitk_ragged_partitions(orc, bits, gs):
    """bf16 partitions whose K ranges start and end inside a 16-byte chunk of
    scales/biases (8 groups) and rows whose group count is not a multiple of 16;
    M covers 1 to 6 row fragments."""
    for M, N, K, S in ((9, 256, 3072, 5), (40, 384, 5120, 3), (85, 200, 7168, 7), (33, 130, 1536, 1)):
        say("ragged partitions", M, N, K, bits, gs, S)
        check_affine(orc, "splitk" if S > 1 else "qmm_t", M, N, K, bits, gs, qi.BF16,
                     seed=2100 + bits * 10 + gs + M, **({"splits": S} if S > 1 else {}))


def test_splitk_many_m_tiles(orc):
    """Split-K with three 128-row tiles of x (M = 300) and a ragged last tile,
    and with three 64-row tiles on 64-column tiles (M = 150, 2/4/8 bits)."""
    check_affine(orc, "splitk", 300, 384, 2048, 4, 64, qi.BF16, seed=1800, splits=4, reruns=1)
    check_affine(orc, "splitk", 300, 200, 2560, 4, 32, qi.F16, seed=1801, splits=5)
    for bits, gs, dt in ((4, 64, qi.BF16), (8, 32, qi.F16), (2, 128, qi.BF16)):
        check_affine(orc, "splitk", 150, 320, 3072, bits, gs, dt, seed=1802 + bits, splits=4)


# ---------------------------------------------------------------- affine sweep (bits x gs x dtype x M)
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dt", [qi.F16, qi.BF16])
def test_config4_sweep(orc, bits, gs, dt):
    N = K = 4096
    for M in (1, 8, 33, 128, 257):
        cols = sample_cols(N, 192, seed=bits * 1000 + gs + M)
        check_affine(orc, "qmm", M, N, K, bits, gs, dt, seed=qi.seed_for(4, bits * 100 + gs + M + dt),
                     cols=cols, bias="exact")


# ---------------------------------------------------------------- Q8_0 / Q4_K
def test_q8_0_config5(orc):
    N, K = 14336, 5120
    say("q8_0", N, K)
    c = qi.q8_0_case(N, K, seed=qi.seed_for(5, 0))
    wb = qmx.words_tensor(c["blocks"], DEV)
    x = torch.from_numpy(c["x"]).to(DEV)
    y = qmx.matvec_q8_0(wb, x)
    y2 = qmx.matvec_q8_0(wb, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert_close(y.cpu().numpy().astype(np.float64), orc.q8_0(c["blocks"], c["x"], N, K), qi.F32, orc, "q8_0")


def test_q4_k_config5(orc):
    N, K = 14336, 5120
    say("q4_k", N, K)
    c = qi.q4_k_case(N, K, seed=qi.seed_for(5, 1))
    wb = qmx.words_tensor(c["blocks"], DEV)
    x = torch.from_numpy(c["x"]).to(DEV)
    y = qmx.matvec_q4_k(wb, x)
    y2 = qmx.matvec_q4_k(wb, x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert_close(y.cpu().numpy().astype(np.float64), orc.q4_k(c["blocks"], c["x"], N, K), qi.F32, orc, "q4_k")


@pytest.mark.parametrize("NK", [(1, 256), (7, 512), (21, 768), (33, 1280), (45, 2560), (130, 4096), (67, 6144),
                                (9, 7936), (40, 8192), (5, 8448), (3, 12800)])
def test_blocks_small_ragged(orc, NK):
    N, K = NK
    say("blocks", N, K)
    c8 = qi.q8_0_case(N, K, seed=1600 + N)
    y = qmx.matvec_q8_0(qmx.words_tensor(c8["blocks"], DEV), torch.from_numpy(c8["x"]).to(DEV))
    assert_close(y.cpu().numpy().astype(np.float64), orc.q8_0(c8["blocks"], c8["x"], N, K), qi.F32, orc)
    c4 = qi.q4_k_case(N, K, seed=1700 + N)
    y = qmx.matvec_q4_k(qmx.words_tensor(c4["blocks"], DEV), torch.from_numpy(c4["x"]).to(DEV))
    assert_close(y.cpu().numpy().astype(np.float64), orc.q4_k(c4["blocks"], c4["x"], N, K), qi.F32, orc)


# ---------------------------------------------------------------- edge cases
def test_empty_and_zero_k(orc):
    say("edge: empty and K=0")
    for route in ("qmv", "qmm_t", "qmm"):
        # M = 0 and N = 0: nothing launched, nothing written
        for M, N in ((0, 64), (16, 0)):
            x = torch.zeros(M, 256, dtype=torch.bfloat16, device=DEV)
            w = torch.zeros(N, 32, dtype=torch.int32, device=DEV)
            s = torch.zeros(N, 4, dtype=torch.bfloat16, device=DEV)
            y = run(route, w, s, s, x, 4, 64)
            assert y.shape == (M, N)
        # K = 0: the sum over no terms is zero
        M = 1 if route == "qmv" else 16
        x = torch.zeros(M, 0, dtype=torch.bfloat16, device=DEV)
        w = torch.zeros(40, 0, dtype=torch.int32, device=DEV)
        s = torch.zeros(40, 0, dtype=torch.bfloat16, device=DEV)
        out = torch.full((M, 40), 7.0, dtype=torch.bfloat16, device=DEV)
        y = run(route, w, s, s, x, 4, 64) if route != "qmm" else qmx.qmm(w, s, s, x, out, bits=4, group_size=64)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y.float()).item() == 0


def test_degenerate_values(orc):
    """All-zero codes give sum_g bias*sum(x); scale 1 / bias 0 with integer x gives the exact
    integer product of the codes."""
    say("edge: degenerate values")
    M, N, K = 16, 128, 1024
    c = qi.affine_case(M, N, K, 4, 64, qi.F32, seed=1800)
    c["w"][:] = 0
    xi = np.random.Generator(np.random.PCG64(1801)).integers(-3, 4, size=(1, K)).astype(np.float32)
    c1 = dict(c, x=xi, M=1, scales=np.ones_like(c["scales"]), biases=np.zeros_like(c["biases"]),
              w=qi.pack_codes(c["codes"], 4))
    w, s, b, x = to_dev(c1)
    y = qmx.qmv(w, s, b, x, bits=4, group_size=64)
    want = xi.astype(np.int64) @ c["codes"].astype(np.int64).T
    assert np.array_equal(y.cpu().numpy().astype(np.float64), want.astype(np.float64))
    for dt in (qi.BF16, qi.F16):
        cz = qi.affine_case(M, N, K, 4, 64, dt, seed=1802)
        cz["w"][:] = 0
        w, s, b, x = to_dev(cz)
        y = qmx.qmm_t(w, s, b, x, bits=4, group_size=64)
        assert_close(out64(y, dt), orc.affine_case(cz), dt, orc, "zero codes")


def test_large_n_and_m(orc):
    # widest configured row count on qmv and a large M on the matrix cores (sampled columns)
    check_affine(orc, "qmv", 1, 27648, 5120, 4, 64, qi.BF16, seed=1900, cols=sample_cols(27648, 512, 1))
    check_affine(orc, "qmm", 1024, 1024, 2048, 4, 64, qi.BF16, seed=1901, cols=sample_cols(1024, 128, 2))


# ---------------------------------------------------------------- batched / strided / odd-offset activations
def _batched_inputs(B, M, N, K, bits, gs, dt, seed, shared_w):
    """B independent problems (each from its own seeded case, or one weight
    set shared by all) as device tensors [B, ...] plus the per-problem cases."""
    cases = [qi.affine_case(M, N, K, bits, gs, dt, seed=seed + (0 if shared_w else i)) for i in range(B)]
    xs = [qi.affine_case(M, N, K, bits, gs, dt, seed=seed + 500 + i)["x"] for i in range(B)]
    for c, x in zip(cases, xs):
        c["x"] = x
    if shared_w:
        w, s, b, _ = to_dev(cases[0])
    else:
        parts = [to_dev(c) for c in cases]
        w, s, b = (torch.stack([p[j] for p in parts]) for j in range(3))
    x = torch.stack([qmx.storage_tensor(c["x"], dt, DEV) for c in cases])
    return cases, w, s, b, x


def _strided(x, kind):
    """The same values as x [B, M, K] in a different layout: rows padded to a
    wider (16-byte aligned) row, or shifted by one element (misaligned)."""
    B, M, K = x.shape
    if kind == "contiguous":
        return x
    pad = 64 if kind == "padded" else 1
    big = torch.zeros((B, M, K + pad + 3), dtype=x.dtype, device=DEV)
    off = 0 if kind == "padded" else 1
    big[:, :, off:off + K] = x
    v = big[:, :, off:off + K]
    assert v.stride(1) == K + pad + 3 and (kind != "odd" or v.data_ptr() % 16 != 0)
    return v


@pytest.mark.parametrize("B,M,N,K,bits,gs,dt,shared,layout", [
    (3, 1, 200, 1024, 4, 64, qi.BF16, False, "contiguous"),   # qmv route, one weight matrix per problem
    (4, 3, 96, 512, 8, 32, qi.F32, True, "padded"),           # qmv route, f32, shared weights, padded rows
    (3, 2, 130, 768, 6, 128, qi.F16, False, "odd"),            # qmv route, odd element offset (copied first)
    (2, 37, 256, 2048, 3, 64, qi.F16, False, "padded"),        # matrix cores, 3-bit, padded rows
    (2, 20, 384, 1024, 4, 64, qi.BF16, True, "odd"),           # matrix cores, odd offset (copied first)
    (2, 16, 256, 4096, 4, 64, qi.BF16, False, "contiguous"),   # split-K across the batch
    (3, 85, 128, 2560, 5, 32, qi.BF16, False, "odd"),          # two M tiles, split-K, odd offset
    (6, 16, 1024, 2048, 4, 64, qi.BF16, False, "padded"),      # 32-column tiles across the batch
    (4, 25, 2048, 1024, 4, 128, qi.F16, True, "odd"),          # 32-column tiles, shared weights, x copied first
    (3, 40, 512, 2048, 8, 64, qi.BF16, True, "padded"),        # 64-column split tiles, shared weights
    (2, 150, 256, 3072, 2, 128, qi.F16, False, "contiguous"),  # 64-column split tiles, three 64-row tiles
])
def test_batched_strided_and_odd_offset(orc, B, M, N, K, bits, gs, dt, shared, layout):
    route = qmx.plan_batched(B, M, N, K, bits, gs, dt, 256)
    say("batched", B, M, N, K, bits, gs, qi.DTYPE_NAMES[dt], shared, layout, route)
    cases, w, s, b, x = _batched_inputs(B, M, N, K, bits, gs, dt, seed=2500 + B + M + bits, shared_w=shared)
    xv = _strided(x, layout)
    y = qmx.qmm_batched(w, s, b, xv, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    got = out64(y, dt)
    for i, c in enumerate(cases):
        ref = orc.affine(c["w"], c["scales"], c["biases"], dt, c["x"], dt, M, N, K, bits, gs)
        assert_close(got[i], ref, dt, orc, what=f"batched problem {i} of {B}, {layout}, route {route}")
    # a second call on the same inputs gives the same bits
    y2 = qmx.qmm_batched(w, s, b, xv, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16) if dt != qi.F32 else y.view(torch.int32),
                       y2.view(torch.int16) if dt != qi.F32 else y2.view(torch.int32))


def test_batched_single_problem_matches_unbatched(orc):
    """A batch of one follows the unbatched plan and gives identical bits."""
    for M, N, K in ((1, 200, 1024), (37, 256, 2048), (16, 256, 4096)):
        say("batch of one", M, N, K)
        c = qi.affine_case(M, N, K, 4, 64, qi.BF16, seed=2600 + M)
        w, s, b, x = to_dev(c)
        assert qmx.plan_batched(1, M, N, K, 4, 64, qi.BF16, 256) == qmx.plan(M, N, K, 4, 64, qi.BF16, 256)
        y1 = qmx.qmm(w, s, b, x, bits=4, group_size=64)
        yb = qmx.qmm_batched(w[None], s[None], b[None], x[None], bits=4, group_size=64)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), yb[0].view(torch.int16))


@pytest.mark.parametrize("M,N,K,bits,gs,dt,layout", [
    (1, 192, 1024, 4, 64, qi.BF16, "contiguous"),     # qmv route
    (5, 160, 768, 3, 32, qi.F16, "odd"),             # qmv route, x copied first
    (24, 256, 2048, 4, 64, qi.BF16, "padded"),        # matrix cores
    (40, 128, 4096, 6, 128, qi.F16, "odd"),          # matrix cores, split-K, x copied first
    (16, 512, 1024, 4, 64, qi.BF16, "padded"),       # matrix cores on 32-column tiles
])
def test_gather_qmm(orc, M, N, K, bits, gs, dt, layout):
    """Problem i takes weight matrix w_index[i] and x matrix x_index[i] (repeated
    and out-of-order picks); each output matches the oracle of its pair."""
    E, X = 3, 2
    w_index = [2, 0, 1, 1, 2, 0, 2]
    x_index = [0, 1, 1, 0, 0, 1, 0]
    B = len(w_index)
    say("gather", M, N, K, bits, gs, qi.DTYPE_NAMES[dt], layout, qmx.plan_batched(B, M, N, K, bits, gs, dt, 256))
    wc = [qi.affine_case(1, N, K, bits, gs, dt, seed=2700 + e) for e in range(E)]
    xc = [qi.affine_case(M, 32, K, 4, gs, dt, seed=2750 + j)["x"] for j in range(X)]
    parts = [to_dev(c) for c in wc]
    w, s, b = (torch.stack([p[j] for p in parts]) for j in range(3))
    x = _strided(torch.stack([qmx.storage_tensor(v, dt, DEV) for v in xc]), layout)
    wi = torch.tensor(w_index, dtype=torch.int32, device=DEV)
    xi = torch.tensor(x_index, dtype=torch.int32, device=DEV)
    y = qmx.gather_qmm(w, s, b, x, wi, xi, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    got = out64(y, dt)
    for i in range(B):
        c = wc[w_index[i]]
        ref = orc.affine(c["w"], c["scales"], c["biases"], dt, xc[x_index[i]], dt, M, N, K, bits, gs)
        assert_close(got[i], ref, dt, orc, what=f"gather problem {i}: W{w_index[i]} x{x_index[i]}")
    # indices outside the ranges are clamped: -3 -> 0, 99 -> E - 1 (and X - 1)
    wi2 = torch.tensor([-3, 99, 1, 1, 2, 0, 2], dtype=torch.int32, device=DEV)
    xi2 = torch.tensor([0, 1, 1, 0, 99, -1, 0], dtype=torch.int32, device=DEV)
    y2 = qmx.gather_qmm(w, s, b, x, wi2, xi2, bits=bits, group_size=gs)
    wi3 = torch.tensor([0, 2, 1, 1, 2, 0, 2], dtype=torch.int32, device=DEV)
    xi3 = torch.tensor([0, 1, 1, 0, 1, 0, 0], dtype=torch.int32, device=DEV)
    y3 = qmx.gather_qmm(w, s, b, x, wi3, xi3, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y3.view(torch.int16))


@pytest.mark.parametrize("N,K,bits,gs,dt,w_index,x_index,layout", [
    # B/E = 12/5: tiles of up to 4 problems; a run of 5 is cut at problem 4
    (200, 1024, 4, 64, qi.BF16, [0, 0, 0, 0, 0, 1, 2, 2, 3, 3, 3, 4], None, "contiguous"),
    # B/E = 2: tiles of up to 2; x picked out of order
    (192, 2048, 4, 64, qi.F16, [0, 0, 1, 1, 1, 2, 3, 3], [3, 0, 2, 1, 3, 0, 1, 2], "contiguous"),
    (96, 512, 8, 32, qi.F32, [0, 0, 0, 1, 1, 1, 1, 2, 2], None, "contiguous"),
    (130, 768, 3, 128, qi.BF16, [1, 1, 1, 0, 0, 2, 2, 2], None, "odd"),     # x copied first
    (64, 1024, 6, 64, qi.F16, [4, 4, 4, 4, 4, 4, 4, 4], [0, 1, 0, 1, 0, 1, 0, 1], "padded"),
    # not sorted: the same results, fewer problems share a tile
    (160, 1024, 4, 64, qi.BF16, [2, 0, 2, 2, 1, 0, 0, 2, 1, 1], None, "contiguous"),
    # out-of-range picks clamp first: -3, 0 -> 0 and 99, 4 -> 4 form runs
    (64, 512, 2, 32, qi.BF16, [-3, 0, 0, 2, 99, 4, 4, 4], None, "contiguous"),
])
def test_gather_sorted_groups(orc, N, K, bits, gs, dt, w_index, x_index, layout):
    """qmx_qmm_gather_sorted at M = 1: consecutive problems on one weight
    matrix share a tile; every output matches the oracle of its (W, x) pair,
    and reruns are bit-identical."""
    E = 5
    B = len(w_index)
    X = 4 if x_index is not None else B
    say("gather_sorted", N, K, bits, gs, qi.DTYPE_NAMES[dt], layout, w_index, x_index)
    wc = [qi.affine_case(1, N, K, bits, gs, dt, seed=2800 + e) for e in range(E)]
    xc = [qi.affine_case(1, 32, K, 4, gs, dt, seed=2850 + j)["x"] for j in range(X)]
    parts = [to_dev(c) for c in wc]
    w, s, b = (torch.stack([p[j] for p in parts]) for j in range(3))
    x = _strided(torch.stack([qmx.storage_tensor(v, dt, DEV) for v in xc]), layout)
    wi = torch.tensor(w_index, dtype=torch.int32, device=DEV)
    xi = torch.tensor(x_index, dtype=torch.int32, device=DEV) if x_index is not None else None
    y = qmx.gather_qmm(w, s, b, x, wi, xi, bits=bits, group_size=gs, sorted_indices=True)
    y2 = qmx.gather_qmm(w, s, b, x, wi, xi, bits=bits, group_size=gs, sorted_indices=True)
    torch.cuda.synchronize()
    got = out64(y, dt)
    for i in range(B):
        we = min(max(w_index[i], 0), E - 1)
        xe = x_index[i] if x_index is not None else i
        c = wc[we]
        ref = orc.affine(c["w"], c["scales"], c["biases"], dt, xc[xe], dt, 1, N, K, bits, gs)
        assert_close(got[i], ref, dt, orc, what=f"sorted gather problem {i}: W{we} x{xe}")
    assert torch.equal(y.view(torch.uint8), y2.view(torch.uint8))


def test_gather_sorted_other_shapes(orc):
    """Shapes the grouping does not cover (M > 1) run as the plain gather."""
    M, N, K, bits, gs, dt = 3, 128, 1024, 4, 64, qi.BF16
    w_index = [0, 0, 1, 1, 1]
    say("gather_sorted M=3", N, K, w_index)
    wc = [qi.affine_case(1, N, K, bits, gs, dt, seed=2900 + e) for e in range(2)]
    xc = [qi.affine_case(M, 32, K, 4, gs, dt, seed=2950 + j)["x"] for j in range(len(w_index))]
    parts = [to_dev(c) for c in wc]
    w, s, b = (torch.stack([p[j] for p in parts]) for j in range(3))
    x = torch.stack([qmx.storage_tensor(v, dt, DEV) for v in xc])
    wi = torch.tensor(w_index, dtype=torch.int32, device=DEV)
    y = qmx.gather_qmm(w, s, b, x, wi, bits=bits, group_size=gs, sorted_indices=True)
    yp = qmx.gather_qmm(w, s, b, x, wi, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), yp.view(torch.int16))
    got = out64(y, dt)
    for i, e in enumerate(w_index):
        c = wc[e]
        ref = orc.affine(c["w"], c["scales"], c["biases"], dt, xc[i], dt, M, N, K, bits, gs)
        assert_close(got[i], ref, dt, orc, what=f"sorted gather M=3 problem {i}")


# ---------------------------------------------------------------- integer activations
def _q8_i8_dev(c):
    return (qmx.words_tensor(c["wq"], DEV), qmx.words_tensor(c["xq"], DEV),
            torch.from_numpy(np.ascontiguousarray(c["wd"])).to(DEV))


@pytest.mark.parametrize("N,K", [(14336, 5120), (1, 32), (7, 256), (33, 1312), (130, 4096)])
def test_q8_i8_matvec(orc, N, K):
    say("q8_i8", N, K)
    c = qi.q8_i8_case(N, K, seed=3000 + N + K)
    wq, xq, wd = _q8_i8_dev(c)
    y = qmx.matvec_q8_i8(wq, xq, wd)
    torch.cuda.synchronize()
    ref = orc.q8_i8(c["wq"], c["xq"], c["wd"], N, K)
    assert_close(y.cpu().numpy().astype(np.float64), ref, qi.F32, orc, what=f"q8_i8 {N}x{K}")
    y2 = qmx.matvec_q8_i8(wq, xq, wd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_q8_i8_integer_exact_and_empty(orc):
    """Unit block scales: every partial sum is an integer below 2^24, so the
    float32 result equals the exact integer product bit for bit; K = 0 gives zeros."""
    N, K = 300, 1024
    say("q8_i8 unit scales", N, K)
    c = qi.q8_i8_case(N, K, seed=3100)
    c["wd"] = np.ones_like(c["wd"])
    wq, xq, wd = _q8_i8_dev(c)
    y = qmx.matvec_q8_i8(wq, xq, wd)
    torch.cuda.synchronize()
    want = c["q"].astype(np.int64) @ c["xq_values"].astype(np.int64)
    assert np.array_equal(y.cpu().numpy().astype(np.int64), want)
    assert np.array_equal(orc.q8_i8(c["wq"], c["xq"], c["wd"], N, K), want.astype(np.float64))
    say("q8_i8 K=0")
    y0 = qmx.matvec_q8_i8(torch.zeros((5, 0), dtype=torch.int32, device=DEV),
                          torch.zeros(0, dtype=torch.int32, device=DEV),
                          torch.zeros((5, 0), dtype=torch.float32, device=DEV),
                          torch.full((5,), 7.0, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(y0, torch.zeros(5, device=DEV))


# ---------------------------------------------------------------- seeded random sweep
def _random_cases(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        bits = int(rng.choice(ALL_BITS))
        gs = int(rng.choice([32, 64, 128]))
        dt = int(rng.choice([qi.F32, qi.F16, qi.BF16]))
        M = int(rng.choice([1, 2, 3, 4, 6, 7, 8, 13, 24, 40, 65, 97, 150]))
        N = int(rng.integers(1, 700))
        K = 128 * int(rng.integers(1, 40))
        route = "qmm" if dt == qi.F32 or rng.random() < 0.5 else str(rng.choice(["qmv", "qmm_t", "splitk"]))
        if route == "splitk" and K // 256 < 2:
            route = "qmm_t"
        out.append((i, M, N, K, bits, gs, dt, route))
    return out


@pytest.mark.parametrize("case", _random_cases(40, 4242), ids=lambda c: f"r{c[0]}")
def test_random_sweep(orc, case):
    """Seeded random shapes, code widths, group sizes, dtypes and routes (ragged N,
    every M tile count), each against the oracle on all outputs."""
    i, M, N, K, bits, gs, dt, route = case
    splits = None
    if route == "splitk":
        splits = int(np.random.Generator(np.random.PCG64(i)).integers(2, min(16, K // 256) + 1))
    check_affine(orc, route, M, N, K, bits, gs, dt, seed=5000 + i, splits=splits)


# ---------------------------------------------------------------- graph capture
def test_graph_replay_matches_eager(orc):
    """The calls captured once in a HIP graph (as bench.py times them) and the
    graph replayed three times, with eager work, output clearing and
    synchronizations between the replays: every replay's outputs equal the
    eager outputs bit for bit, and the eager outputs match the oracle."""
    say("graph replay: qmv, split-K qmm, unsplit qmm, sorted gather, q8_0, q4_k")
    dt = qi.BF16
    cv = qi.affine_case(1, 200, 1024, 4, 64, dt, seed=3100)
    cs = qi.affine_case(22, 384, 2048, 4, 64, dt, seed=3101)
    cu = qi.affine_case(40, 256, 256, 3, 32, dt, seed=3102)
    args = {k: to_dev(c) for k, c in (("v", cv), ("s", cs), ("u", cu))}
    route_s = qmx.plan(22, 384, 2048, 4, 64, dt)
    assert route_s[0] == "qmm_t_splitk", route_s
    ws = torch.empty(max(1, qmx.qmm_workspace_bytes(22, 384, 2048, 4, 64, dt) // 4), dtype=torch.float32,
                     device=DEV)
    wc = [qi.affine_case(1, 128, 512, 4, 64, dt, seed=3110 + e) for e in range(3)]
    gp = [to_dev(c) for c in wc]
    gw, gs_, gb = (torch.stack([p[j] for p in gp]) for j in range(3))
    gx = torch.stack([qmx.storage_tensor(qi.affine_case(1, 32, 512, 4, 64, dt, seed=3120 + j)["x"], dt, DEV)
                      for j in range(6)])
    gi_host = [0, 0, 1, 1, 2, 2]
    gi = torch.tensor(gi_host, dtype=torch.int32, device=DEV)
    c8 = qi.q8_0_case(64, 1024, seed=3130)
    c4 = qi.q4_k_case(64, 1024, seed=3131)
    b8, x8 = qmx.words_tensor(c8["blocks"], DEV), torch.from_numpy(c8["x"]).to(DEV)
    b4, x4 = qmx.words_tensor(c4["blocks"], DEV), torch.from_numpy(c4["x"]).to(DEV)
    outs = {
        "v": torch.empty((1, 200), dtype=torch.bfloat16, device=DEV),
        "s": torch.empty((22, 384), dtype=torch.bfloat16, device=DEV),
        "u": torch.empty((40, 256), dtype=torch.bfloat16, device=DEV),
        "g": torch.empty((6, 1, 128), dtype=torch.bfloat16, device=DEV),
        "q8": torch.empty(64, dtype=torch.float32, device=DEV),
        "q4": torch.empty(64, dtype=torch.float32, device=DEV),
    }

    def step():
        qmx.qmm(*args["v"], outs["v"], bits=4, group_size=64)
        qmx.qmm(*args["s"], outs["s"], bits=4, group_size=64, workspace=ws)
        qmx.qmm(*args["u"], outs["u"], bits=3, group_size=32)
        qmx.gather_qmm(gw, gs_, gb, gx, gi, None, outs["g"], bits=4, group_size=64, sorted_indices=True)
        qmx.matvec_q8_0(b8, x8, outs["q8"])
        qmx.matvec_q4_k(b4, x4, outs["q4"])

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}
    # the eager outputs against the oracle
    for k, c, m in (("v", cv, 1), ("s", cs, 22), ("u", cu, 40)):
        assert_close(out64(eager[k], dt), orc.affine_case(c), dt, orc, what=f"graph eager {k}")
    for i, e in enumerate(gi_host):
        c = wc[e]
        xi = qi.affine_case(1, 32, 512, 4, 64, dt, seed=3120 + i)["x"]
        ref = orc.affine(c["w"], c["scales"], c["biases"], dt, xi, dt, 1, 128, 512, 4, 64)
        assert_close(out64(eager["g"], dt)[i], ref, dt, orc, what=f"graph eager gather {i}")
    assert_close(eager["q8"].cpu().numpy().astype(np.float64), orc.q8_0(c8["blocks"], c8["x"], 64, 1024), qi.F32,
                 orc, "graph eager q8_0")
    assert_close(eager["q4"].cpu().numpy().astype(np.float64), orc.q4_k(c4["blocks"], c4["x"], 64, 1024), qi.F32,
                 orc, "graph eager q4_k")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    junk = torch.randn(512, 512, device=DEV)
    for rep in range(3):
        for v in outs.values():
            v.zero_()
        junk = junk @ junk.T / 512.0             # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v.view(torch.uint8), eager[k].view(torch.uint8)), f"replay {rep}: {k}"


@pytest.mark.parametrize("sorted_indices", [False, True])
def test_gather_bench_size(orc, sorted_indices):
    """The gather workload's own size: 16 problems over 8 weight matrices of
    2048 x 4096 (4-bit gs 64 bf16, M = 1), each matrix picked twice, in random
    order or ordered by matrix; sampled columns of every problem against the
    oracle."""
    B, E, N, K = 16, 8, 2048, 4096
    g = torch.Generator(device="cpu")
    g.manual_seed(3200)
    picks = (torch.randperm(B, generator=g) % E)
    if sorted_indices:
        picks = torch.sort(picks).values
    w_index = picks.tolist()
    say("gather bench size", B, E, N, K, "sorted" if sorted_indices else "random", w_index)
    wc = [qi.affine_case(1, N, K, 4, 64, qi.BF16, seed=3210 + e) for e in range(E)]
    xc = [qi.affine_case(1, 32, K, 4, 64, qi.BF16, seed=3230 + j)["x"] for j in range(B)]
    parts = [to_dev(c) for c in wc]
    w, s, b = (torch.stack([p[j] for p in parts]) for j in range(3))
    x = torch.stack([qmx.storage_tensor(v, qi.BF16, DEV) for v in xc])
    wi = torch.tensor(w_index, dtype=torch.int32, device=DEV)
    y = qmx.gather_qmm(w, s, b, x, wi, bits=4, group_size=64, sorted_indices=sorted_indices)
    torch.cuda.synchronize()
    got = out64(y, qi.BF16)
    cols = sample_cols(N, 192, seed=3240)
    for i, e in enumerate(w_index):
        c = wc[e]
        ref = orc.affine(c["w"], c["scales"], c["biases"], qi.BF16, xc[i], qi.BF16, 1, N, K, 4, 64, cols=cols)
        assert_close(got[i][:, cols], ref, qi.BF16, orc, what=f"gather bench-size problem {i}: W{e}")


@pytest.mark.parametrize("M,N", [(257, 4096), (384, 4096), (512, 1024), (300, 1024)])
def test_qmm_large_m_tilings(orc, M, N):
    """The policy above M = 192: 128-row tiles split in 2 (M = 257), 64-row
    tiles unsplit (M = 384) and 64-row tiles split (N = 1024), sampled
    columns of every row against the oracle, reruns bit-identical."""
    route = qmx.plan(M, N, 4096, 4, 64, qi.BF16)
    say("large-M tiling", M, N, route)
    check_affine(orc, "qmm", M, N, 4096, 4, 64, qi.BF16, seed=3300 + M + N, cols=sample_cols(N, 96, M + N),
                 reruns=1)
