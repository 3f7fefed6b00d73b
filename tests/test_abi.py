"""The C ABI on the CPU: the library loads, exports every declared entry point,
rejects bad arguments before any HIP call, and the dispatch policy table.

No compute call is made here (no GPU in this tier); argument errors return
before the library touches the HIP runtime.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmx.h")

import matmul_affine_qmv_amd as qmx  # noqa: E402

if not os.path.exists(qmx.LIB_PATH):
    pytest.skip("libqmx.so not built", allow_module_level=True)

OK, ENULL, ESHAPE, EBITS, EGROUP, EDTYPE, EALIGN, EWS, ESPLITS = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmx_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"qmx_qmv", "qmx_qmm_t", "qmx_qmm_t_splitk", "qmx_matvec_q8_0", "qmx_matvec_q4_k",
            "qmx_qmm", "qmx_plan"} <= set(names)
    raw = ctypes.CDLL(qmx.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(qmx._EXPORTS), "binding and header disagree"


def test_calibration_library_exports_its_header():
    """libqmx_calib.so (streaming-read, copy, matrix-core and empty kernels used
    beside the measurements) exports exactly what include/qmx_calib.h declares."""
    from matmul_affine_qmv_amd import calib
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "qmx_calib.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(qmxc_[a-z0-9_]+)\s*\(", text)))
    assert names == sorted(calib.EXPORTS)
    raw = ctypes.CDLL(calib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    L = calib.lib()
    # argument errors return before any HIP call
    assert L.qmxc_read(None, 16, None, 0, 1, None) == -1
    assert L.qmxc_read(16, 17, 16, 0, 1, None) == -1
    assert L.qmxc_copy(16, 32, 16, 0, None) == -1
    assert L.qmxc_mfma(None, 1, 1, 32, None) == -1
    assert L.qmxc_mfma(16, 1, 1, 8, None) == -1
    assert L.qmxc_empty(0, None) == -1


def test_version_and_strerror():
    assert qmx.api_version() == 1
    for code in range(-10, 1):
        assert qmx.strerror(code) and qmx.strerror(code) != "unknown status"
    assert qmx.strerror(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x10002)


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0


# The calls below pass placeholder pointers that must never reach a kernel.  They
# are meant for the CPU tier; on a machine with a GPU a validation slip would
# launch a kernel on them, so there they are skipped.
fake_ptr_test = pytest.mark.skipif(_gpu_visible(), reason="placeholder pointers: CPU-only checks")


def qmv(w=FAKE, s=FAKE, b=FAKE, x=FAKE, o=FAKE, M=1, N=64, K=4096, bits=4, gs=64, dt=BF16):
    return qmx.lib().qmx_qmv(w, s, b, x, o, M, N, K, bits, gs, dt, None)


def qmm_t(w=FAKE, s=FAKE, b=FAKE, x=FAKE, o=FAKE, M=16, N=64, K=4096, bits=4, gs=64, dt=BF16):
    return qmx.lib().qmx_qmm_t(w, s, b, x, o, M, N, K, bits, gs, dt, None)


def splitk(splits=2, ws=FAKE, wsb=1 << 30, M=16, N=64, K=4096, bits=4, gs=64, dt=BF16, x=FAKE, w=FAKE):
    return qmx.lib().qmx_qmm_t_splitk(w, FAKE, FAKE, x, FAKE, M, N, K, bits, gs, dt, splits, ws, wsb, None)


@fake_ptr_test
def test_qmv_validation():
    for bad in (0, 7, 9, 16):
        assert qmv(bits=bad) == EBITS
    for good in (1, 2, 3, 4, 5, 6, 8):   # accepted widths reach the empty-problem exit
        assert qmv(bits=good, M=0, w=None, x=None, o=None) == OK
    assert qmv(gs=16) == EGROUP
    assert qmv(K=4000) == EGROUP           # not a multiple of 64
    assert qmv(dt=7) == EDTYPE
    assert qmv(M=-1) == ESHAPE
    assert qmv(N=-4) == ESHAPE
    assert qmv(K=96, gs=32, bits=2) == ESHAPE   # 192 bits per row is not whole 16-byte chunks
    assert qmv(o=None) == ENULL
    assert qmv(w=None) == ENULL
    assert qmv(x=None) == ENULL
    assert qmv(w=ODD) == EALIGN
    assert qmv(x=ODD) == EALIGN
    # empty problems succeed without touching the device or the pointers
    assert qmv(M=0, w=None, x=None, o=None) == OK
    assert qmv(N=0, w=None, x=None, o=None) == OK


@fake_ptr_test
def test_qmm_t_validation():
    assert qmm_t(dt=F32) == EDTYPE
    assert qmm_t(K=4032) == ESHAPE          # K % 128 != 0 (but K % 64 == 0)
    assert qmm_t(bits=7) == EBITS
    assert qmm_t(bits=5, M=0, w=None) == OK
    assert qmm_t(gs=256) == EGROUP
    assert qmm_t(s=None) == ENULL
    assert qmm_t(x=ODD) == EALIGN
    assert qmm_t(M=0, w=None) == OK


@fake_ptr_test
def test_splitk_validation():
    assert splitk(splits=1) == ESPLITS
    assert splitk(splits=17) == ESPLITS
    assert splitk(splits=3, K=512) == ESPLITS      # 512/3 < 256 columns per partition
    assert splitk(splits=2, K=512, ws=None) == EWS
    assert splitk(splits=4, wsb=4 * 16 * 64 * 4 - 4) == EWS
    assert splitk(splits=4, ws=ctypes.c_void_p(0x10004)) == EWS
    assert qmx.splitk_workspace_bytes(85, 2048, 4) == 4 * 85 * 2048 * 4
    assert qmx.splitk_workspace_bytes(-1, 2, 2) == 0


@fake_ptr_test
def test_partials_and_accumulate_validation():
    L = qmx.lib()

    def parts(splits=4, ws=FAKE, wsb=1 << 30, M=16, N=64, K=4096, dt=BF16):
        return L.qmx_qmm_t_partials(FAKE, FAKE, FAKE, FAKE, M, N, K, 4, 64, dt, splits, ws, wsb, None)

    assert parts(splits=1) == ESPLITS
    assert parts(splits=17) == ESPLITS
    assert parts(splits=3, K=512) == ESPLITS
    assert parts(ws=None) == EWS
    assert parts(wsb=4 * 16 * 64 * 4 - 1) == EWS
    assert parts(dt=F32) == EDTYPE
    assert parts(M=0, ws=None) == OK
    acc = L.qmx_splitk_accumulate
    assert acc(FAKE, FAKE, 4, 4, 1, BF16, None) == ESPLITS
    assert acc(FAKE, FAKE, 4, 4, 17, BF16, None) == ESPLITS
    assert acc(FAKE, FAKE, 4, 4, 2, F32, None) == EDTYPE
    assert acc(FAKE, FAKE, -1, 4, 2, BF16, None) == ESHAPE
    assert acc(None, FAKE, 4, 4, 2, BF16, None) == EWS
    assert acc(ctypes.c_void_p(0x10008), FAKE, 4, 4, 2, BF16, None) == EWS
    assert acc(FAKE, None, 4, 4, 2, BF16, None) == ENULL
    assert acc(FAKE, ctypes.c_void_p(0x10001), 4, 4, 2, BF16, None) == EALIGN
    assert acc(None, None, 0, 4, 2, BF16, None) == OK


@fake_ptr_test
def test_block_validation():
    L = qmx.lib()
    assert L.qmx_matvec_q8_0(FAKE, FAKE, FAKE, 16, 48, None) == EGROUP
    assert L.qmx_matvec_q8_0(FAKE, FAKE, None, 16, 64, None) == ENULL
    assert L.qmx_matvec_q8_0(ODD, FAKE, FAKE, 16, 64, None) == EALIGN
    assert L.qmx_matvec_q8_0(FAKE, FAKE, FAKE, -1, 64, None) == ESHAPE
    assert L.qmx_matvec_q8_0(None, None, None, 0, 64, None) == OK
    assert L.qmx_matvec_q4_k(FAKE, FAKE, FAKE, 16, 128, None) == EGROUP
    assert L.qmx_matvec_q4_k(FAKE, ODD, FAKE, 16, 256, None) == EALIGN
    assert L.qmx_matvec_q4_k(None, None, None, 0, 256, None) == OK


@pytest.mark.parametrize("M,N,K,dtype,route,splits", [
    (1, 4096, 4096, BF16, "qmv", 1),
    (4, 4096, 4096, BF16, "qmm_t", 1),              # 16-column tiles: 6.8 us against 8.0 us for qmv
    (7, 4096, 4096, BF16, "qmm_t", 1),                # a second qmv pass costs more than 32-column tiles
    (16, 4096, 4096, F32, "qmv", 1),                 # float32 never takes the matrix cores
    (16, 4096, 4096, BF16, "qmm_t", 1),              # 128 32-column tiles instead of 32 x 8 partitions
    (16, 4096, 4096, F16, "qmm_t", 1),
    (16, 4096, 256, BF16, "qmm_t", 1),               # K < 1024 stays unsplit
    (16, 4096, 768, BF16, "qmm_t", 1),
    (16, 4096, 1024, BF16, "qmm_t", 1),              # 2 narrow blocks against 2 blocks + the accumulate
    (22, 2048, 2048, BF16, "qmm_t", 1),              # 64 32-column tiles, 4 blocks each
    (22, 2048, 8192, BF16, "qmm_t_splitk", 8),       # 16 narrow blocks: too long; 32 64-column tiles x 8
    (40, 2048, 2048, BF16, "qmm_t_splitk", 8),       # M > 32: 32 64-column tiles x 8 partitions
    (85, 2048, 10752, BF16, "qmm_t_splitk", 4),      # 2 M tiles of 64 rows x 32 64-column tiles
    (128, 4096, 4096, BF16, "qmm_t_splitk", 2),      # 2 M tiles of 64 rows x 64 64-column tiles
    (33, 4096, 14336, BF16, "qmm_t_splitk", 4),
    (56, 5120, 17408, BF16, "qmm_t_splitk", 3),      # floor(256 / 80 64-column tiles)
    (512, 4096, 4096, BF16, "qmm_t", 1),             # 64-row tiles: 8 M tiles x 32 N tiles fill 256 CUs
    (1024, 4096, 4096, BF16, "qmm_t", 1),            # 128-row tiles: 8 x 32
    (512, 1024, 4096, BF16, "qmm_t_splitk", 4),      # 64-row tiles, 8 x 8 = 64 tiles: 4 partitions
    (257, 4096, 4096, BF16, "qmm_t_splitk", 2),      # 128-row tiles: 3 x 32 split 2 = 192 groups (64-row: 160)
    (384, 4096, 4096, BF16, "qmm_t", 1),             # 64-row tiles: 6 x 32 = 192 groups, as many as 3 x 32 split 2
    (257, 16384, 4096, F16, "qmm_t", 1),             # 3 x 128 tiles >= 256 CUs
    (8, 4096, 4096, F16, "qmm_t", 1),
    (16, 14336, 4096, BF16, "qmm_t", 1),             # two rounds of 448 narrow tiles, 8 blocks each
    (16, 16384, 8192, BF16, "qmm_t_splitk", 2),      # ... but not at 16 blocks per round
    (16, 4096, 4032, BF16, "qmv", 1),                # K % 128 != 0 -> qmv
    (2, 14336, 5120, BF16, "qmv", 1),                # M = 2..7: qmv while its vector work is small
    (4, 14336, 5120, BF16, "qmm_t", 1),              # ... the matrix route once it is not
    (7, 27648, 5120, BF16, "qmm_t", 1),
    (5, 5120, 5120, F16, "qmm_t", 1),
    (4, 5120, 5120, BF16, "qmm_t", 1),               # measured: 32-column tiles 9.5 us, qmv 12.1 us
    (7, 2048, 2048, BF16, "qmm_t", 1),              # 16-column tiles: 5.0 us against 6.1 us for qmv
    (7, 14336, 5120, F32, "qmv", 1),                 # float32 stays on qmv at every M
    (16, 1024, 4096, BF16, "qmm_t", 1),              # 64 16-column tiles: 6.6 us against 8.1 split in 16
    (16, 4096, 8192, BF16, "qmm_t", 1),              # 16 blocks of 16 columns: 10.4 us against 12.6 split in 8
    (16, 1024, 8192, BF16, "qmm_t_splitk", 16),      # ... 9.6 us against 9.2 split in 16
    (2, 2048, 8192, BF16, "qmv", 1),                 # M = 2 stays on qmv where 16-column tiles apply
    (5, 2048, 2048, BF16, "qmm_t", 1),               # from M = 3 they take the matrix route (5.0 against 6.0 us)
    (4, 2048, 8192, BF16, "qmm_t_splitk", 8),        # qmv walks a long K slowly
])
def test_plan_table(M, N, K, dtype, route, splits):
    assert qmx.plan(M, N, K, 4, 64, dtype, num_cus=256) == (route, splits)


def test_plan_narrow_tiles_take_2_4_8_bit_codes():
    """The 32-column tiles read 2-, 4- and 8-bit codes; the other widths keep the
    128-column tiles and their split-K partitions (capped at K / 256)."""
    for bits in (2, 8):
        assert qmx.plan(16, 4096, 4096, bits, 64, BF16, num_cus=256) == ("qmm_t", 1)
        assert qmx.plan(16, 4096, 4096, bits, 128, BF16, num_cus=256) == ("qmm_t", 1)
    for bits in (2, 4, 8):   # gs 32: two group epilogues per wave and block; 16-column tiles
        # within 2 blocks of the split plan (8 against 4 x 0.7 here)
        assert qmx.plan(16, 4096, 4096, bits, 32, BF16, num_cus=256) == ("qmm_t", 1)
    # ... and the split plan beyond that, or where 32-column tiles would be needed
    assert qmx.plan(16, 2048, 2048, 4, 32, BF16, num_cus=256) == ("qmm_t", 1)       # 5.4 against 7.1 us
    assert qmx.plan(16, 1024, 4096, 4, 32, BF16, num_cus=256) == ("qmm_t_splitk", 16)  # 7.3 against 7.8
    assert qmx.plan(16, 4096, 8192, 4, 32, BF16, num_cus=256) == ("qmm_t_splitk", 4)   # 11.6 against 12.6
    assert qmx.plan(16, 14336, 4096, 4, 32, BF16, num_cus=256) == ("qmm_t_splitk", 2)  # 16.3 against 19.8
    assert qmx.plan(4, 4096, 4096, 4, 32, BF16, num_cus=256) == ("qmv", 1)   # M = 2..7 rule fitted at gs 64
    for bits in (1, 3, 5, 6):
        assert qmx.plan(16, 4096, 4096, bits, 64, BF16, num_cus=256) == ("qmm_t_splitk", 8)
        assert qmx.plan(16, 4096, 1024, bits, 64, BF16, num_cus=256) == ("qmm_t_splitk", 4)
    # K not a multiple of 512 keeps them too
    assert qmx.plan(16, 4096, 1152, 4, 64, BF16, num_cus=256)[0] == "qmm_t_splitk"


def test_plan_64_column_split_needs_staged_scales():
    """64-column split tiles take half the partitions only where their LDS holds
    the longest partition's scales and biases: at (17408, 5120, 56) the 8-bit
    work-group has room for 6 chunks, the partition needs 14, so the 128-column
    plan (6 partitions) stays; 2- and 4-bit work-groups hold 15."""
    assert qmx.plan(56, 5120, 17408, 8, 64, BF16, num_cus=256) == ("qmm_t_splitk", 6)
    for bits in (2, 4):
        assert qmx.plan(56, 5120, 17408, bits, 64, BF16, num_cus=256) == ("qmm_t_splitk", 3)
    assert qmx.plan(56, 5120, 17408, 4, 32, F16, num_cus=256) == ("qmm_t_splitk", 6)   # 23 chunks at gs 32
    assert qmx.plan(128, 4096, 4096, 8, 64, BF16, num_cus=256) == ("qmm_t_splitk", 2)  # 4 + 2 chunks fit
    assert qmx.plan(85, 2048, 10752, 8, 64, BF16, num_cus=256) == ("qmm_t_splitk", 4)


def test_plan_respects_split_limits():
    for K in (512, 768, 1024, 2048, 14336):
        for N in (128, 1024, 4096):
            route, s = qmx.plan(16, N, K, 4, 64, BF16, 256)
            if route == "qmm_t_splitk":
                assert 2 <= s <= 16 and K // s >= 256
    with pytest.raises(qmx.QmxError):
        qmx.plan(16, 4096, 96, 2, 32, F32, 256)      # qmv route cannot take 192-bit rows
    with pytest.raises(qmx.QmxError):
        qmx.plan(1, 4096, 4096, 7, 64, BF16, 256)      # 7-bit codes are not a supported width
    for bits in (1, 3, 5, 6):                          # the other widths take the same routes; their split
        assert qmx.plan(1, 4096, 4096, bits, 64, BF16, 256) == ("qmv", 1)      # plans stay on 128-column tiles
        assert qmx.plan(40, 4096, 4096, bits, 64, BF16, 256) == ("qmm_t_splitk", 8)
    assert qmx.plan(40, 4096, 4096, 4, 64, BF16, 256) == ("qmm_t_splitk", 4)   # 64 64-column tiles x 4


def test_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, dtype=torch.bfloat16)
    w = torch.zeros(8, 8, dtype=torch.int32)
    s = torch.zeros(8, 1, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        qmx.qmv(w, s, s, x, bits=4, group_size=64)


@fake_ptr_test
def test_batched_validation():
    L = qmx.lib()

    def bat(B=2, M=4, N=64, K=512, ws=128, sbs=64, xs=2048, xr=512, bits=4, gs=64, dt=BF16, w=FAKE, x=FAKE,
            o=FAKE, work=None, wb=0):
        return L.qmx_qmm_batched(w, FAKE, FAKE, x, o, B, M, N, K, ws, sbs, xs, xr, bits, gs, dt, work, wb, None)

    assert bat(B=-1) == ESHAPE
    assert bat(B=65536) == ESHAPE
    assert bat(xr=511) == ESHAPE             # rows shorter than K
    assert bat(ws=-4) == ESHAPE
    assert bat(ws=6) == EALIGN               # weight matrices must stay 16-byte aligned
    assert bat(bits=7) == EBITS
    assert bat(K=500) == EGROUP
    assert bat(B=0, w=None, x=None, o=None) == OK
    assert bat(M=0, w=None, x=None, o=None) == OK
    # workspace sizes: partials only when the plan splits, plus the copy of a misaligned x
    wsb = L.qmx_qmm_batched_workspace_bytes
    assert wsb(2, 4, 64, 512, 4, 64, BF16, FAKE, 2048, 512) == 0          # qmv route, aligned x
    assert wsb(2, 4, 64, 512, 4, 64, BF16, ODD, 2048, 512) == 2 * 4 * 512 * 2
    assert wsb(2, 4, 64, 512, 4, 64, BF16, FAKE, 2048, 513) == 2 * 4 * 512 * 2   # odd row stride


def test_batched_plan_counts_every_problem():
    # one problem of (M=40, N=256, K=4096) has 2 tiles: 16 partitions; 8 of them: 16 tiles, 16 partitions;
    # 200 of them fill the chip without a split
    assert qmx.plan_batched(1, 40, 256, 4096, 4, 64, BF16, 256) == qmx.plan(40, 256, 4096, 4, 64, BF16, 256)
    r8, s8 = qmx.plan_batched(8, 40, 256, 4096, 4, 64, BF16, 256)
    r1, s1 = qmx.plan_batched(1, 40, 256, 4096, 4, 64, BF16, 256)
    assert r8 == r1 == "qmm_t_splitk" and s8 <= s1
    assert qmx.plan_batched(200, 40, 256, 4096, 4, 64, BF16, 256) == ("qmm_t", 1)
    # at M = 16 the 32-column tiles of 8 problems (64 of them) take the batch unsplit
    assert qmx.plan_batched(1, 16, 256, 4096, 4, 64, BF16, 256)[0] == "qmm_t_splitk"
    assert qmx.plan_batched(8, 16, 256, 4096, 4, 64, BF16, 256) == ("qmm_t", 1)
    assert qmx.plan_batched(8, 1, 4096, 4096, 4, 64, BF16, 256) == ("qmv", 1)


@fake_ptr_test
def test_gather_validation():
    L = qmx.lib()

    for fn in (L.qmx_qmm_gather, L.qmx_qmm_gather_sorted):
        def gat(B=3, nw=2, nx=2, M=4, N=64, K=512, w=FAKE, x=FAKE, o=FAKE, wi=FAKE, xi=FAKE):
            return fn(w, FAKE, FAKE, x, o, wi, xi, nw, nx, B, M, N, K, 128, 64, 2048, 512, 4, 64, BF16,
                      None, 0, None)

        assert gat(nw=0) == ESHAPE                # a non-empty batch needs at least one weight matrix
        assert gat(nx=-1) == ESHAPE
        assert gat(M=1, nw=0) == ESHAPE
        assert gat(B=0, w=None, x=None, o=None, wi=None, xi=None) == OK
    assert L.qmx_qmm_gather_workspace_bytes(3, 2, 4, 64, 512, 4, 64, BF16, ODD, 2048, 512) == 2 * 4 * 512 * 2


@fake_ptr_test
def test_q8_i8_validation():
    f = qmx.lib().qmx_matvec_q8_i8
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 48, None) == EGROUP      # K not a multiple of 32
    assert f(FAKE, FAKE, FAKE, FAKE, -1, 64, None) == ESHAPE
    assert f(ODD, FAKE, FAKE, FAKE, 8, 64, None) == EALIGN       # packed weights need 16-byte alignment
    assert f(FAKE, FAKE, ctypes.c_void_p(0x10001), FAKE, 8, 64, None) == EALIGN
    assert f(FAKE, None, FAKE, FAKE, 8, 64, None) == ENULL
    assert f(None, None, None, FAKE, 0, 64, None) == OK          # empty output
