"""A seeded sweep of prefill and recurrent calls against the fp64 oracle.

Each case draws its own combination of the features the fixed parity tests
cover one at a time: I/O dtype, head count, packed batches with empty,
one-token, chunk-boundary and ragged sequences, the single-sequence launch
(no cu_seqlens), nonzero or absent initial states, mild, split and extreme
decay recipes, in-kernel L2Norm on raw q/k, and workspaces that force the
prefill into windows of a few chunk slots. Batches whose mean length is at
most two chunks (or four, with at least 256 (sequence, head) pairs: a mode
of its own) take the short-sequence carry, other batches with more than 32
pairs the two-tile carry; batches of sequences no longer than 64 tokens
also go through the recurrent path. Tolerances as in the
other parity tests (max |o - o_ref| / max |o_ref|, relative Frobenius error
of the final state)."""
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
    return dict(lengths=lengths, H=H, seed=7100 + i, io=io, decay=decay,
                h0_std=h0_std, qk="raw" if l2norm else "unit"), \
        dict(l2norm=l2norm, single=single, window=window)


def _slot_bytes(H, io):
    return H * (40960 * (2 if io == "bf16" else 4) + 128 * 4)


def _oracle(p, l2norm):
    q, k = (recurrent.l2norm(p.q), recurrent.l2norm(p.k)) if l2norm else (p.q, p.k)
    return recurrent.forward(q, k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)


def _check(p, o, hf, ro, rh, what):
    tol_o, tol_s = TOL[p.io]
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
    args = (dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
            None if p.h0 is None else dev(p.h0),
            None if opt["single"] else dev(p.cu_seqlens, torch.int32))
    ws = None
    if opt["window"] is not None:
        nbytes = (kda.chunk_fwd_workspace_min_bytes(p.N, p.T, p.H, dt) +
                  (opt["window"] - 1) * _slot_bytes(p.H, p.io))
        ws = kda.alloc_workspace(p.N, p.T, p.H, dt, "cuda", nbytes=nbytes)
    o, hf = kda.chunk_fwd(*args, workspace=ws, qk_l2norm=opt["l2norm"])
    torch.cuda.synchronize()
    ro, rh = _oracle(p, opt["l2norm"])
    _check(p, host(o), host(hf), ro, rh, "chunk_fwd")
    if max(wargs["lengths"]) <= 64:
        o2, h2 = kda.recurrent_fwd(*args[:6], dev(p.cu_seqlens, torch.int32), n_seqs=p.N,
                                   qk_l2norm=opt["l2norm"])
        torch.cuda.synchronize()
        _check(p, host(o2), host(h2), ro, rh, "recurrent_fwd")
