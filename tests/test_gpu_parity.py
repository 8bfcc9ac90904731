"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle.

Small shapes span several chunks and a ragged tail; the tolerance measures
are max|o - o_ref| / max|o_ref| and the relative Frobenius error of the final
state (fp32 I/O: 1e-4 / 1e-4; bf16 I/O: 2e-2 / 1e-2).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_50_amd import kda, workloads  # noqa: E402
from oracle import recurrent  # noqa: E402
from tests.kda_testutil import TOL, dev, host, io_dtype, rel_fro_err, rel_max_err  # noqa: E402

pytestmark = pytest.mark.gpu


def _run_prefill(p, h0=True, cu=True):
    dt = io_dtype(p.io)
    o, hf = kda.chunk_fwd(
        dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
        dev(p.h0) if (h0 and p.h0 is not None) else None,
        dev(p.cu_seqlens, torch.int32) if cu else None)
    torch.cuda.synchronize()
    return host(o), host(hf)


def _check_prefill(p, o, hf, heads=None):
    sel = slice(None) if heads is None else heads
    ro, rh = recurrent.forward(p.q[:, sel], p.k[:, sel], p.v[:, sel], p.log_alpha[:, sel],
                               p.beta[:, sel], None if p.h0 is None else p.h0[:, sel],
                               p.cu_seqlens)
    tol_o, tol_s = TOL[p.io]
    eo = rel_max_err(o[:, sel], ro)
    es = rel_fro_err(hf[:, sel], rh)
    print(f"o err {eo:.3e} (tol {tol_o}), state err {es:.3e} (tol {tol_s})")
    assert np.isfinite(o).all() and np.isfinite(hf).all()
    assert eo <= tol_o, eo
    assert es <= tol_s, es
    return eo, es


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 333])
def test_prefill_single_sequence(io, T):
    p = workloads.make_prefill([T], H=3, seed=T, io=io, h0_std=0.05)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_packed_with_empty_and_ragged(io):
    lens = [70, 0, 1, 128, 5, 64, 0, 190]
    p = workloads.make_prefill(lens, H=2, seed=7, io=io, h0_std=0.05)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)
    # empty sequences keep their initial state exactly
    np.testing.assert_array_equal(hf[1], p.h0[1])
    np.testing.assert_array_equal(hf[6], p.h0[6])


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_null_h0_equals_zero_h0(io):
    p = workloads.make_prefill([150], H=2, seed=8, io=io)
    o1, h1 = _run_prefill(p, h0=False, cu=False)
    p.h0 = np.zeros((1, 2, 128, 128), np.float32)
    o2, h2 = _run_prefill(p, h0=True, cu=True)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)
    _check_prefill(p, o1, h1)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_strong_decay(io):
    """cfg-2 style split decay: half the channels lose e^-16..e^-64 per chunk."""
    p = workloads.make_prefill([300], H=2, seed=9, io=io, decay="split", h0_std=0.02)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_extreme_decay_exact_fallback(io):
    """log alpha = -6 per token on some channels makes in-block decay ratios
    exceed e^44; those diagonal blocks take the exact per-element path."""
    p = workloads.make_prefill([200], H=2, seed=10, io=io, h0_std=0.05)
    p.log_alpha[:, :, :16] = -6.0
    p.log_alpha[:, :, 100:104] = -30.0
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)


def test_config0_tiny_fp32():
    p = workloads.config(0).prefill()
    o, hf = _run_prefill(p, cu=False)
    _check_prefill(p, o, hf)


def test_config1_prefill_8k_sampled_heads():
    p = workloads.config(1).prefill()
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf, heads=[0, 7, 19, 31])


# ------------------------------------------------------------- decode
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_steps_small(io):
    N, H = 5, 3
    S0 = workloads.make_decode_state(N, H, seed=3, std=0.05)
    S = dev(S0)
    ref = S0.astype(np.float64)
    dt = io_dtype(io)
    for step in range(4):
        d = workloads.make_decode_step(N, H, seed=3, step=step, io=io)
        o = kda.decode_step(dev(d.q, dt), dev(d.k, dt), dev(d.v, dt), dev(d.log_alpha),
                            dev(d.beta), S)
        torch.cuda.synchronize()
        ro, ref = recurrent.decode_step(d.q, d.k, d.v, d.log_alpha, d.beta, ref)
        tol_o, tol_s = TOL[io]
        assert rel_max_err(host(o), ro) <= tol_o
        assert rel_fro_err(host(S), ref) <= tol_s


def test_phases_equal_full_call_and_deterministic():
    """Phases 0, 1, 2 in order equal kda_chunk_fwd bitwise; repeated calls are
    bitwise identical (no atomics, fixed reduction orders)."""
    p = workloads.make_prefill([100, 300], H=4, seed=21, io="bf16", h0_std=0.05)
    bf = torch.bfloat16
    args = (dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha), dev(p.beta),
            dev(p.h0), dev(p.cu_seqlens, torch.int32))
    pre = kda.Prefill(*args)
    o1, h1 = (x.clone() for x in pre.run())
    for ph in range(3):
        pre.run_phase(ph)
    torch.cuda.synchronize()
    assert torch.equal(pre.o, o1) and torch.equal(pre.h_final, h1)
    o3, h3 = pre.run()
    torch.cuda.synchronize()
    assert torch.equal(o3, o1) and torch.equal(h3, h1)
