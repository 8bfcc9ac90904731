"""The prefill over windows of chunk slots (a workspace smaller than the
call's blocks): each window's intra-chunk kernel then carry, with the state
of a sequence crossing a window boundary handed over through the
workspace's state area. The per-chunk arithmetic does not depend on the
window, so every windowed run must equal the one-window run bit for bit;
one case is also checked against the fp64 oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_50_amd import kda, workloads  # noqa: E402
from oracle import recurrent  # noqa: E402
from tests.kda_testutil import TOL, dev, host, io_dtype, rel_fro_err, rel_max_err  # noqa: E402,F401

pytestmark = pytest.mark.gpu


def _args(p, cu=True):
    dt = io_dtype(p.io)
    return (dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
            None if p.h0 is None else dev(p.h0),
            dev(p.cu_seqlens, torch.int32) if cu else None)


def _slot_bytes(H, io):
    """Workspace bytes per chunk slot: one intermediate block per head."""
    return H * (40960 * (2 if io == "bf16" else 4) + 128 * 4)


def _workspace(p, window_slots):
    """A workspace holding `window_slots` chunk slots per window (None: the
    recommended size, one window for these calls)."""
    dt = io_dtype(p.io)
    nbytes = None
    if window_slots is not None:
        nbytes = (kda.chunk_fwd_workspace_min_bytes(p.N, p.T, p.H, dt) +
                  (window_slots - 1) * _slot_bytes(p.H, p.io))
    return kda.alloc_workspace(p.N, p.T, p.H, dt, "cuda", nbytes=nbytes)


def _run(p, window_slots=None, cu=True):
    o, hf = kda.chunk_fwd(*_args(p, cu), workspace=_workspace(p, window_slots))
    torch.cuda.synchronize()
    return o, hf


def _same(a, b):
    return torch.equal(a.view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.view(torch.int32 if b.dtype == torch.float32 else torch.int16))


CASES = {
    # one sequence: the single-sequence launch path, pipelined one-tile carry
    "single_bf16": (dict(lengths=[1000], H=4, seed=601, io="bf16", h0_std=0.05), False),
    # packed with empty and one-token sequences, nonzero initial states
    "packed_bf16": (dict(lengths=[300, 0, 1, 129, 64, 700, 0], H=3, seed=602, io="bf16",
                         h0_std=0.05), True),
    "packed_f32": (dict(lengths=[200, 65, 0, 130], H=2, seed=603, io="f32", h0_std=0.05), True),
    # more than 32 (sequence, head) pairs: two column tiles per carry workgroup
    "two_tile": (dict(lengths=list(np.random.default_rng(5).integers(130, 400, 20)), H=2,
                      seed=604, io="bf16", h0_std=0.05), True),
    # mean length up to two chunks: the short-sequence carry
    "short": (dict(lengths=list(np.random.default_rng(6).integers(0, 129, 40)), H=2, seed=605,
                   io="bf16", h0_std=0.05), True),
    # strong decays: exact diagonal blocks in every window
    "extreme": (dict(lengths=[333, 70], H=2, seed=606, io="bf16", decay="extreme",
                     h0_std=0.05), True),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("window", [1, 2, 3, 7])
def test_windowed_equals_one_window(name, window):
    spec, cu = CASES[name]
    p = workloads.make_prefill(**spec)
    print(f"{name}: lengths {np.diff(p.cu_seqlens).tolist()}, window {window}", flush=True)
    o1, h1 = _run(p, None, cu)
    ow, hw = _run(p, window, cu)
    assert _same(o1, ow), "outputs differ"
    assert _same(h1, hw), "final states differ"


def test_windowed_against_oracle():
    """Windows of two chunk slots over a packed batch, against the oracle."""
    p = workloads.make_prefill([500, 3, 0, 260, 1], H=2, seed=607, io="bf16", h0_std=0.05)
    o, hf = _run(p, 2)
    ro, rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)
    eo, es = rel_max_err(host(o), ro), rel_fro_err(host(hf), rh)
    print(f"o err {eo:.3e}, state err {es:.3e}")
    assert eo <= TOL["bf16"][0] and es <= TOL["bf16"][1]


def test_windowed_all_empty_sequences():
    """T = 0: every sequence copies its initial state, whatever the window."""
    p = workloads.make_prefill([0, 0, 0], H=2, seed=608, io="bf16", h0_std=0.05)
    o, hf = _run(p, 1)
    assert torch.equal(hf.cpu(), torch.from_numpy(p.h0))


def test_windowed_in_place_continuation():
    """h_final = h0 (in place) across windows: the state area, not h0, carries
    a sequence between windows, so the result equals a separate h_final."""
    p = workloads.make_prefill([400, 250], H=2, seed=609, io="bf16", h0_std=0.05)
    args = _args(p)
    ws = _workspace(p, 3)
    o_ref, h_ref = kda.chunk_fwd(*args, workspace=ws)
    h = args[5].clone()
    o, _ = kda.chunk_fwd(*args[:5], h, args[6], h_final=h, workspace=ws)
    torch.cuda.synchronize()
    assert _same(o, o_ref) and _same(h, h_ref)
