"""Prefill with bfloat16 initial and final states (KDA_FLAG_STATE_BF16), the
state format of the "L2 Deep Distill" page's serving notes.

The call widens h0 to fp32, carries the state in fp32 and rounds it once into
h_final, so for a bf16-exact h0 it must give exactly the outputs of the fp32
state call and h_final = round_to_nearest_even(h_final of the fp32 call), on
every carry form (pipelined one-tile, two-tile, short-sequence, fp32 I/O) and
with windows. Against the fp64 oracle it meets the bf16 I/O tolerances.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_50_amd import kda, workloads  # noqa: E402
from oracle import recurrent  # noqa: E402
from tests.kda_testutil import TOL, dev, host, io_dtype, rel_fro_err, rel_max_err  # noqa: E402

pytestmark = pytest.mark.gpu
bf = torch.bfloat16


def _bf16_h0(p):
    """p's h0 rounded to bf16 (device bf16 tensor) and the same values as a
    host fp64 array."""
    h0 = dev(p.h0).to(bf)
    return h0, host(h0)


def _args(p):
    dt = io_dtype(p.io)
    cu = dev(p.cu_seqlens, torch.int32) if p.N > 1 else None
    return (dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta)), cu


def _batch(name):
    rng = np.random.default_rng(70)
    if name == "one sequence":
        return workloads.make_prefill([333], H=3, seed=71, io="bf16", h0_std=0.05)
    if name == "two-tile":
        return workloads.make_prefill(
            [int(x) for x in rng.integers(150, 400, size=18)] + [0, 1, 64, 129], H=2, seed=72,
            io="bf16", h0_std=0.05)
    if name == "short":
        return workloads.make_prefill(
            [int(x) for x in rng.integers(0, 140, size=40)] + [0, 1, 63, 64, 65, 128, 129],
            H=3, seed=73, io="bf16", h0_std=0.05)
    return workloads.make_prefill([1, 200, 0, 65], H=2, seed=74, io="f32", h0_std=0.05)


@pytest.mark.parametrize("name", ["one sequence", "two-tile", "short", "fp32 I/O"])
def test_bf16_state_equals_rounded_fp32_state_call(name):
    p = _batch(name)
    (q, k, v, la, b), cu = _args(p)
    h0b, _ = _bf16_h0(p)
    o32, h32 = kda.chunk_fwd(q, k, v, la, b, h0b.float(), cu)
    o16, h16 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    torch.cuda.synchronize()
    assert h16.dtype == bf and h16.shape == h32.shape
    assert torch.equal(o16, o32), name
    assert torch.equal(h16, h32.to(bf)), name


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bf16_state_prefill_matches_oracle(io):
    p = workloads.make_prefill([70, 0, 1, 128, 5, 190], H=2, seed=75, io=io, h0_std=0.05)
    (q, k, v, la, b), cu = _args(p)
    h0b, h0h = _bf16_h0(p)
    o, hf = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    torch.cuda.synchronize()
    ro, rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, h0h, p.cu_seqlens)
    assert rel_max_err(host(o), ro) <= TOL["bf16"][0]
    assert rel_fro_err(host(hf), rh) <= TOL["bf16"][1]
    # empty sequences keep their (bf16) initial state exactly
    assert torch.equal(hf[1], h0b[1])


def test_bf16_state_in_place_and_null_h0():
    p = workloads.make_prefill([200, 77], H=3, seed=76, io="bf16", h0_std=0.05)
    (q, k, v, la, b), cu = _args(p)
    h0b, _ = _bf16_h0(p)
    o1, h1 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    state = h0b.clone()
    o2, h2 = kda.chunk_fwd(q, k, v, la, b, state, cu, h_final=state, state_dtype=bf)
    torch.cuda.synchronize()
    assert h2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, state)
    o3, h3 = kda.chunk_fwd(q, k, v, la, b, None, cu, state_dtype=bf)
    o4, h4 = kda.chunk_fwd(q, k, v, la, b, torch.zeros_like(h0b), cu, state_dtype=bf)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(h3, h4)


def test_bf16_state_windows_equal_one_window():
    """Sequences crossing window boundaries carry their state through the
    workspace in fp32: the bf16 h_final is the same as with one window."""
    p = workloads.make_prefill([700, 130, 1000], H=2, seed=77, io="bf16", h0_std=0.05)
    (q, k, v, la, b), cu = _args(p)
    h0b, _ = _bf16_h0(p)
    o1, h1 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    small = kda.alloc_workspace(p.N, p.T, p.H, bf, q.device,
                                nbytes=kda.chunk_fwd_workspace_min_bytes(p.N, p.T, p.H, bf)
                                + 2 * p.H * 82432)
    o2, h2 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, workspace=small, state_dtype=bf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_bf16_state_noalloc_equals_chunk_fwd():
    p = workloads.make_prefill([300, 64], H=2, seed=78, io="bf16", h0_std=0.05)
    (q, k, v, la, b), cu = _args(p)
    h0b, _ = _bf16_h0(p)
    o1, h1 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    o2, h2 = kda.chunk_fwd_noalloc(q, k, v, la, b, h0b, cu, state_dtype=bf)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_bf16_state_prefill_then_recurrent_decode():
    """The serving flow with the state kept in bf16 between calls: a prefill
    of 300 tokens, then 8 single-token recurrent steps updating the bf16 state
    in place, against the fp64 oracle over all 308 tokens."""
    T0, steps, H = 300, 8, 4
    p = workloads.make_prefill([T0 + steps], H=H, seed=79, io="bf16", h0_std=0.05)
    h0b, h0h = _bf16_h0(p)
    q, k, v = (dev(x, bf) for x in (p.q, p.k, p.v))
    la, b = dev(p.log_alpha), dev(p.beta)
    o_pre, state = kda.chunk_fwd(q[:T0], k[:T0], v[:T0], la[:T0], b[:T0], h0b, state_dtype=bf)
    outs = [host(o_pre)]
    for t in range(T0, T0 + steps):
        o_t, _ = kda.recurrent_fwd(q[t:t + 1], k[t:t + 1], v[t:t + 1], la[t:t + 1], b[t:t + 1],
                                   state, None, n_seqs=1, state_dtype=bf, h_final=state)
        outs.append(host(o_t))
    torch.cuda.synchronize()
    ro, rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, h0h)
    assert rel_max_err(np.concatenate(outs), ro) <= TOL["bf16"][0]
    assert rel_fro_err(host(state), rh) <= TOL["bf16"][1]


@pytest.mark.parametrize("T", [12, 300])
def test_forward_switch_with_bf16_state(T):
    """kda.forward keeps the state in bf16 on both of its paths."""
    p = workloads.make_prefill([T], H=4, seed=80 + T, io="bf16", h0_std=0.05)
    h0b, h0h = _bf16_h0(p)
    (q, k, v, la, b), _ = _args(p)
    o, hf = kda.forward(q, k, v, la, b, h0b, max_seqlen=T, state_dtype=bf)
    torch.cuda.synchronize()
    assert hf.dtype == bf
    ro, rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, h0h)
    assert rel_max_err(host(o), ro) <= TOL["bf16"][0]
    assert rel_fro_err(host(hf), rh) <= TOL["bf16"][1]


def test_bf16_state_dtype_checked_by_the_binding():
    p = workloads.make_prefill([64], H=1, seed=81, io="bf16", h0_std=0.05)
    (q, k, v, la, b), _ = _args(p)
    with pytest.raises(TypeError):
        kda.chunk_fwd(q, k, v, la, b, dev(p.h0), state_dtype=bf)   # fp32 h0 for a bf16 state
    with pytest.raises(TypeError):
        kda.chunk_fwd(q, k, v, la, b, dev(p.h0).to(bf))            # bf16 h0 for an fp32 state


@pytest.mark.parametrize("T,H,N", [(8192, 32, 1), (8192, 32, 4)])
def test_bf16_state_full_size_equals_rounded_fp32_state_call(T, H, N):
    """At the 8K x 32-head size (every carry workgroup of the one-tile and,
    with four sequences, the two-tile form), the bf16-state call is the
    fp32-state call with its final state rounded."""
    p = workloads.make_prefill([T // N] * N, H=H, seed=82 + N, io="bf16", h0_std=0.02)
    (q, k, v, la, b), cu = _args(p)
    h0b, _ = _bf16_h0(p)
    o32, h32 = kda.chunk_fwd(q, k, v, la, b, h0b.float(), cu)
    o16, h16 = kda.chunk_fwd(q, k, v, la, b, h0b, cu, state_dtype=bf)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32)
    assert torch.equal(h16, h32.to(bf))
