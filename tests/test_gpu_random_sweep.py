"""Seeded sweeps against the fp64 oracle: prefill and recurrent calls, and
decode steps.

Each case draws its own combination of the features the fixed parity tests
cover one at a time: I/O dtype, head count, packed batches with empty,
one-token, chunk-boundary and ragged sequences, the single-sequence launch
(no cu_seqlens), nonzero or absent initial states in fp32 or bf16, mild,
split and extreme decay recipes, in-kernel L2Norm on raw q/k, and workspaces
that force the prefill into windows of a few chunk slots. Batches whose mean length is at
most two chunks (or four, with at least 256 (sequence, head) pairs: a mode
of its own) take the short-sequence carry, other batches with more than 32
pairs the two-tile carry; batches of sequences no longer than 64 tokens
also go through the recurrent path. Tolerances as in the
other parity tests (max |o - o_ref| / max |o_ref|, relative Frobenius error
of the final state). The decode sweep draws sequence and head counts (so
both decode slice widths run), I/O dtype, fp32 or bf16 states and in-kernel
L2Norm, and runs one to three steps with the state carried on the device."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gated_delta_rule_50_amd import kda, workloads  # noqa: E402
from oracle import recurrent  # noqa: E402
from tests.kda_testutil import TOL, dev, host, io_dtype, rel_fro_err, rel_max_err  # noqa: E402

pytestmark = pytest.mark.gpu

N_CASES = 128


def _draw_case(i):
    """Case i of the sweep: a dict of workload arguments and call options,
    from its own seeded stream."""
    rng = np.random.default_rng(7000 + i)
    io = "bf16" if rng.random() < 0.7 else "f32"
    H = int(rng.choice([1, 2, 3, 4, 5, 8]))
    N = int(rng.integers(1, 7))
    if rng.random() < 0.2:
        N = int(rng.integers(9, 17))   # many pairs: two-tile carry at H >= 3
    kinds = rng.random(N)
    lengths = []
    for u in kinds:
        if u < 0.1:
            lengths.append(0)
        elif u < 0.2:
            lengths.append(1)
        elif u < 0.35:
            lengths.append(int(rng.choice([63, 64, 65, 128])))
        else:
            lengths.append(int(rng.integers(2, 400)))
    decay = str(rng.choice(["mild", "mild", "mild", "split", "split", "extreme"]))
    l2norm = bool(rng.random() < 0.2)
    h0_std = None if rng.random() < 0.3 else 0.05
    single = N == 1 and rng.random() < 0.5
    window = None
    if rng.random() < 0.4:
        window = int(rng.integers(1, 6))
    if rng.random() < 0.12:
        # at least 256 (sequence, head) pairs with a mean of two to four
        # chunks: the short-sequence carry's many-pair case
        H = 16
        N = int(rng.integers(16, 25))
        lengths = [int(x) for x in rng.integers(100, 300, size=N)]
        single = False
    # drawn last, so the other draws of every case stay as they were
    bf16_state = bool(rng.random() < 0.25)
    return dict(lengths=lengths, H=H, seed=7100 + i, io=io, decay=decay,
                h0_std=h0_std, qk="raw" if l2norm else "unit"), \
        dict(l2norm=l2norm, single=single, window=window, bf16_state=bf16_state)


def _slot_bytes(H, io):
    return H * (40960 * (2 if io == "bf16" else 4) + 128 * 4)


def _oracle(p, l2norm):
    q, k = (recurrent.l2norm(p.q), recurrent.l2norm(p.k)) if l2norm else (p.q, p.k)
    return recurrent.forward(q, k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)


def _check(p, o, hf, ro, rh, what, bf16_state=False):
    # a bf16 state sets the error, whatever the I/O dtype
    tol_o, tol_s = TOL["bf16" if bf16_state else p.io]
    assert np.isfinite(o).all() and np.isfinite(hf).all(), what
    if p.T == 0:
        return
    eo, es = rel_max_err(o, ro), rel_fro_err(hf, rh)
    print(f"{what}: o err {eo:.3e} (tol {tol_o}), state err {es:.3e} (tol {tol_s})")
    assert eo <= tol_o and es <= tol_s, (what, eo, es)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case_against_oracle(i):
    wargs, opt = _draw_case(i)
    p = workloads.make_prefill(**wargs)
    print(f"case {i}: lengths {wargs['lengths']} H {p.H} io {p.io} decay {wargs['decay']} "
          f"h0 {p.h0 is not None} {opt}")
    dt = io_dtype(p.io)
    sdt = torch.bfloat16 if opt["bf16_state"] else torch.float32
    if opt["bf16_state"] and p.h0 is not None:
        p.h0 = workloads.round_bf16(p.h0)   # the oracle starts from the bf16 state
    args = (dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
            None if p.h0 is None else dev(p.h0, sdt),
            None if opt["single"] else dev(p.cu_seqlens, torch.int32))
    ws = None
    if opt["window"] is not None:
        nbytes = (kda.chunk_fwd_workspace_min_bytes(p.N, p.T, p.H, dt) +
                  (opt["window"] - 1) * _slot_bytes(p.H, p.io))
        ws = kda.alloc_workspace(p.N, p.T, p.H, dt, "cuda", nbytes=nbytes)
    o, hf = kda.chunk_fwd(*args, workspace=ws, qk_l2norm=opt["l2norm"], state_dtype=sdt)
    torch.cuda.synchronize()
    assert hf.dtype == sdt
    ro, rh = _oracle(p, opt["l2norm"])
    _check(p, host(o), host(hf), ro, rh, "chunk_fwd", opt["bf16_state"])
    if max(wargs["lengths"]) <= 64:
        o2, h2 = kda.recurrent_fwd(*args[:6], dev(p.cu_seqlens, torch.int32), n_seqs=p.N,
                                   qk_l2norm=opt["l2norm"], state_dtype=sdt)
        torch.cuda.synchronize()
        _check(p, host(o2), host(h2), ro, rh, "recurrent_fwd", opt["bf16_state"])


N_DECODE = 32


def _draw_decode(i):
    """Decode case i: (io, N, H, steps, bf16 state, L2Norm), from its own
    seeded stream. Small pair counts take the 16-column decode slices, bf16
    states the 64-column ones."""
    rng = np.random.default_rng(8000 + i)
    io = "bf16" if rng.random() < 0.6 else "f32"
    N = int(rng.choice([1, 2, 3, 5, 8, 17, 40]))
    H = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    steps = int(rng.integers(1, 4))
    bf16_state = bool(rng.random() < 0.3)
    l2norm = bool(rng.random() < 0.25)
    return io, N, H, steps, bf16_state, l2norm


@pytest.mark.parametrize("i", range(N_DECODE))
def test_random_decode_against_oracle(i):
    """A few decode steps per case, the state carried on the device and in
    fp64 by the oracle; fp32 states through kda_decode_step (or, with
    L2Norm, kda_recurrent_fwd on one token), bf16 states through
    kda_recurrent_fwd (rounded after every step, state tolerance 1e-2)."""
    io, N, H, steps, bf16_state, l2norm = _draw_decode(i)
    print(f"decode case {i}: io {io} N {N} H {H} steps {steps} bf16 state {bf16_state} "
          f"l2norm {l2norm}")
    S0 = workloads.make_decode_state(N, H, 8100 + i)
    if bf16_state:
        S0 = workloads.round_bf16(S0)
    S = dev(S0, torch.bfloat16 if bf16_state else torch.float32)
    ref = S0.astype(np.float64)
    dt = io_dtype(io)
    tol_o, tol_s = TOL[io]
    if bf16_state:   # the rounded state sets the error, whatever the I/O dtype
        tol_o, tol_s = TOL["bf16"]
    for step in range(steps):
        d = workloads.make_decode_step(N, H, 8200 + i, step, io=io,
                                       qk="raw" if l2norm else "unit")
        args = (dev(d.q, dt), dev(d.k, dt), dev(d.v, dt), dev(d.log_alpha), dev(d.beta))
        if bf16_state or l2norm:
            o, _ = kda.recurrent_fwd(*args, S, n_seqs=N, qk_l2norm=l2norm,
                                     state_dtype=S.dtype, h_final=S)
        else:
            o = kda.decode_step(*args, S)
        torch.cuda.synchronize()
        q, k = (recurrent.l2norm(d.q), recurrent.l2norm(d.k)) if l2norm else (d.q, d.k)
        ro, ref = recurrent.decode_step(q, k, d.v, d.log_alpha, d.beta, ref)
        eo = rel_max_err(host(o).reshape(ro.shape), ro)
        es = rel_fro_err(S.float().cpu().numpy().astype(np.float64), ref)
        print(f"  step {step}: o err {eo:.3e} (tol {tol_o}), state err {es:.3e} (tol {tol_s})")
        assert np.isfinite(host(o)).all()
        assert eo <= tol_o and es <= tol_s, (step, eo, es)
