"""qmx_qmm_t_splitk_noalloc (float32 partials in the library's per-device
scratch array) against qmx_qmm_t_splitk (caller workspace), through the C ABI,
on consecutive calls that reuse the scratch array, the later ones smaller.
Needs a gfx950 GPU; every case prints its name before it touches the GPU.
"""
import ctypes
import sys

import pytest

import qmx_inputs as qi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import matmul_affine_qmv_amd as qmx  # noqa: E402

DEV = "cuda:0"
TORCH_DT = {qi.F16: torch.float16, qi.BF16: torch.bfloat16}
FAKE = ctypes.c_void_p(0x1000)


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def noalloc(w, s, b, x, out, M, N, K, bits, gs, dt, splits):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return qmx.lib().qmx_qmm_t_splitk_noalloc(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(),
                                              out.data_ptr(), M, N, K, bits, gs, dt, splits, stream)


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # config-3 shape at the policy's split, then smaller problems on the same scratch array
    for M, N, K, bits, gs, dt, S, seed in ((56, 5120, 17408, 4, 64, qi.BF16, 6, 2101),
                                           (22, 2048, 2048, 4, 64, qi.BF16, 8, 2102),
                                           (37, 160, 768, 2, 32, qi.F16, 3, 2103)):
        say("noalloc split-K", M, N, K, bits, gs, dt, S)
        c = qi.affine_case(M, N, K, bits, gs, dt, seed=seed)
        w, s, b, x = (qmx.words_tensor(c["w"], DEV), qmx.storage_tensor(c["scales"], dt, DEV),
                      qmx.storage_tensor(c["biases"], dt, DEV), qmx.storage_tensor(c["x"], dt, DEV))
        out = torch.full((M, N), float("nan"), dtype=TORCH_DT[dt], device=DEV)
        rc = noalloc(w, s, b, x, out, M, N, K, bits, gs, dt, S)
        assert rc == 0, qmx.strerror(rc)
        ref = qmx.qmm_t_splitk(w, s, b, x, bits=bits, group_size=gs, splits=S)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_noalloc_rejects_partials_beyond_its_scratch():
    """Sizes past QMX_NOALLOC_SCRATCH_BYTES are refused before anything runs."""
    L = qmx.lib()
    limit = 16 << 20
    assert qmx.splitk_workspace_bytes(64, 16384, 4) == limit
    assert L.qmx_qmm_t_splitk_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 16384, 4096, 4, 64, qi.BF16, 5,
                                      None) == -11
    assert L.qmx_qmm_t_splitk_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 85, 14336, 5120, 4, 64, qi.BF16, 16,
                                      None) == -11
    assert "scratch" in qmx.strerror(-11)
    # argument errors come first for problems that fit
    assert L.qmx_qmm_t_splitk_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 4096, 4, 64, qi.BF16, 1,
                                      None) == -8
    # an empty problem succeeds without touching the device
    assert L.qmx_qmm_t_splitk_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 4096, 4, 64, qi.BF16, 2, None) == 0
