"""The achievable-rate probes bench.py reports beside its rooflines do the
work they are timed for: the copy copies, the in-place update rewrites every
element, and the read, MFMA and FMA loops run to completion (their results
stay out of memory unless a value the data never takes turns up)."""
import ctypes

import pytest

torch = pytest.importorskip("torch")

from probes.build import LIB as CEIL_LIB  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probes():
    if not CEIL_LIB.exists():
        pytest.fail(f"{CEIL_LIB} is not built")
    P = ctypes.CDLL(str(CEIL_LIB))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    P.kdab_read.argtypes = [vp, i64, vp, i32, vp]
    P.kdab_copy.argtypes = [vp, vp, i64, i32, i32, vp]
    P.kdab_rmw.argtypes = [vp, i64, i32, vp]
    P.kdab_mfma.argtypes = [vp, i64, i32, vp]
    P.kdab_valu.argtypes = [vp, i64, i32, vp]
    return P


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("n", [4, 1000, 262148])   # ragged against 256 lanes x 4 unrolled
def test_copy_and_update(probes, nt, n):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = torch.randn(n * 4, device="cuda")
    b = torch.full((n * 4 + 64,), -7.0, device="cuda")
    assert probes.kdab_copy(_p(a), _p(b), n * 16, nt, 37, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(b[:n * 4], a) and bool((b[n * 4:] == -7.0).all())
    want = a * 0.5 + 0.25
    assert probes.kdab_rmw(_p(a), n * 16, 37, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(a, want)


def test_read_and_compute_loops_leave_the_sink(probes):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    a = torch.randn(1 << 16, device="cuda")
    sink = torch.zeros(256, device="cuda")
    assert probes.kdab_read(_p(a), a.numel() * 4, _p(sink), 64, st) == 0
    assert probes.kdab_mfma(_p(sink), 16, 64, st) == 0
    assert probes.kdab_valu(_p(sink), 16, 64, st) == 0
    torch.cuda.synchronize()
    assert not sink.any()
