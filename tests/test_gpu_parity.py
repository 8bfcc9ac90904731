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


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_extreme_recipe_packed(io):
    """The "extreme" gate recipe (half the channels at log alpha in [-4, -3],
    so every 16-token diagonal block takes the exact path) on a packed batch
    with ragged tails and nonzero initial states."""
    p = workloads.make_prefill([300, 17, 64, 0, 129], H=4, seed=11, io=io, decay="extreme",
                               h0_std=0.05)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)


def _check_prefill_l2norm(p, o, hf):
    ro, rh = recurrent.forward(recurrent.l2norm(p.q), recurrent.l2norm(p.k), p.v,
                               p.log_alpha, p.beta, p.h0, p.cu_seqlens)
    tol_o, tol_s = TOL[p.io]
    eo, es = rel_max_err(o, ro), rel_fro_err(hf, rh)
    print(f"o err {eo:.3e} (tol {tol_o}), state err {es:.3e} (tol {tol_s})")
    assert np.isfinite(o).all() and np.isfinite(hf).all()
    assert eo <= tol_o and es <= tol_s, (eo, es)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_in_kernel_l2norm(io):
    """Un-normalised q, k (norm ~ 11) with the L2Norm flag against the oracle
    on l2norm(q), l2norm(k) in fp64; packed, with ragged tails."""
    p = workloads.make_prefill([70, 1, 130, 0, 64], H=2, seed=40, io=io, h0_std=0.05, qk="raw")
    dt = io_dtype(p.io)
    o, hf = kda.chunk_fwd(dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha),
                          dev(p.beta), dev(p.h0), dev(p.cu_seqlens, torch.int32),
                          qk_l2norm=True)
    torch.cuda.synchronize()
    _check_prefill_l2norm(p, host(o), host(hf))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_prefill_l2norm_exact_fallback(io):
    """The exact diagonal-block path (in-block decay ratios past e^44) with
    the L2Norm flag: its re-read rows take the same scales."""
    p = workloads.make_prefill([200], H=2, seed=41, io=io, h0_std=0.05, qk="raw")
    p.log_alpha[:, :, :16] = -6.0
    dt = io_dtype(p.io)
    o, hf = kda.chunk_fwd(dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha),
                          dev(p.beta), dev(p.h0), dev(p.cu_seqlens, torch.int32),
                          qk_l2norm=True)
    torch.cuda.synchronize()
    _check_prefill_l2norm(p, host(o), host(hf))


def test_prefill_l2norm_flag_on_unit_inputs():
    """On unit-norm inputs the flag changes results only at rounding level,
    and the two forward paths agree with it set."""
    p = workloads.make_prefill([150, 9], H=2, seed=42, io="f32", h0_std=0.05)
    args = (dev(p.q), dev(p.k), dev(p.v), dev(p.log_alpha), dev(p.beta), dev(p.h0),
            dev(p.cu_seqlens, torch.int32))
    o1, h1 = kda.chunk_fwd(*args)
    o2, h2 = kda.chunk_fwd(*args, qk_l2norm=True)
    o3, h3 = kda.recurrent_fwd(*args, qk_l2norm=True)
    torch.cuda.synchronize()
    assert rel_max_err(host(o2), host(o1)) <= 1e-5 and rel_fro_err(host(h2), host(h1)) <= 1e-5
    assert rel_max_err(host(o3), host(o2)) <= 1e-4 and rel_fro_err(host(h3), host(h2)) <= 1e-4


def test_config0_tiny_fp32():
    p = workloads.config(0).prefill()
    o, hf = _run_prefill(p, cu=False)
    _check_prefill(p, o, hf)


def test_config1_prefill_8k_all_heads():
    p = workloads.config(1).prefill()
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)


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


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_bound_decode_static_buffers(io):
    """A Decode bound once to static token buffers, refilled before each run,
    matches the oracle step by step and decode_step on fresh tensors bit for
    bit."""
    N, H, steps = 4, 3, 5
    dt = io_dtype(io)
    S0 = workloads.make_decode_state(N, H, seed=6, std=0.05)
    S_bound, S_free = dev(S0), dev(S0)
    ref = S0.astype(np.float64)
    bufs = dict(q=torch.empty((N, H, 128), dtype=dt, device="cuda"),
                k=torch.empty((N, H, 128), dtype=dt, device="cuda"),
                v=torch.empty((N, H, 128), dtype=dt, device="cuda"),
                la=torch.empty((N, H, 128), dtype=torch.float32, device="cuda"),
                beta=torch.empty((N, H), dtype=torch.float32, device="cuda"))
    step_fn = kda.Decode(bufs["q"], bufs["k"], bufs["v"], bufs["la"], bufs["beta"], S_bound)
    tol_o, tol_s = TOL[io]
    for step in range(steps):
        d = workloads.make_decode_step(N, H, seed=6, step=step, io=io)
        toks = (dev(d.q, dt), dev(d.k, dt), dev(d.v, dt), dev(d.log_alpha), dev(d.beta))
        for buf, t in zip(bufs.values(), toks):
            buf.copy_(t)
        o_bound = step_fn.run()
        o_free = kda.decode_step(*toks, S_free)
        torch.cuda.synchronize()
        assert torch.equal(o_bound, o_free) and torch.equal(S_bound, S_free), step
        ro, ref = recurrent.decode_step(d.q, d.k, d.v, d.log_alpha, d.beta, ref)
        assert rel_max_err(host(o_bound), ro) <= tol_o
        assert rel_fro_err(host(S_bound), ref) <= tol_s


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


# ------------------------------------------- many (sequence, head) pairs
# Once the one-tile carry workgroups (eight per pair) outnumber the 256 CUs,
# the carry runs two column tiles per workgroup; these batches take that
# path (more than 32 pairs), with ragged, one-token and empty sequences.
def _many_pairs_batch(seed, io="bf16"):
    """More (sequence, head) pairs than one round of one-tile carry
    workgroups, sequences long enough on average (> 128 tokens) for the
    pipelined carry."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(150, 400, size=18)] + [0, 1, 64, 129]
    p = workloads.make_prefill(lengths, H=2, seed=seed, io=io, h0_std=0.05)
    assert p.T > 128 * p.N
    return p


def _short_batch(seed, n=40, H=3):
    """A batch of short sequences (mean at most 128 tokens: the short-sequence
    carry) with the edge lengths 0, 1, 63, 64, 65, 128 and 129."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(0, 140, size=n)] + [0, 1, 63, 64, 65, 128, 129]
    p = workloads.make_prefill(lengths, H=H, seed=seed, io="bf16", h0_std=0.05)
    assert p.T <= 128 * p.N
    return p


def test_short_sequence_carry_matches_oracle():
    p = _short_batch(65)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)
    rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)[1]
    for n in range(p.N):   # every sequence's final state, the empty ones included
        assert rel_fro_err(hf[n], rh[n]) <= TOL[p.io][1], n


def test_short_sequence_carry_equals_pipelined_bitwise():
    """The short-sequence carry (the batch) and the pipelined carry (each
    sequence alone) do the same arithmetic per tile and chunk."""
    p = _short_batch(66, n=12, H=2)
    o, hf = _run_prefill(p)
    bf = torch.bfloat16
    cu = p.cu_seqlens
    for n in range(p.N):
        s, e = int(cu[n]), int(cu[n + 1])
        if e == s:
            continue
        on, hn = kda.chunk_fwd(dev(p.q[s:e], bf), dev(p.k[s:e], bf), dev(p.v[s:e], bf),
                               dev(p.log_alpha[s:e]), dev(p.beta[s:e]), dev(p.h0[n:n + 1]))
        torch.cuda.synchronize()
        assert np.array_equal(host(on), o[s:e]) and np.array_equal(host(hn)[0], hf[n]), n


def _short_many_pairs_batch(seed):
    """At least 256 (sequence, head) pairs with a mean length between two and
    four chunks: the short-sequence carry's second case."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(100, 330, size=60)] + [0, 1, 64, 256]
    p = workloads.make_prefill(lengths, H=4, seed=seed, io="bf16", h0_std=0.05)
    assert 128 * p.N < p.T <= 256 * p.N and p.N * p.H >= 256
    return p


def test_short_carry_many_pairs_matches_oracle():
    p = _short_many_pairs_batch(67)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)
    rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)[1]
    for n in range(p.N):
        assert rel_fro_err(hf[n], rh[n]) <= TOL[p.io][1], n


def test_short_carry_many_pairs_equals_pipelined_bitwise():
    """Sequences of the many-pair batch run alone (pipelined carry) give the
    same bits as inside the batch (short-sequence carry)."""
    p = _short_many_pairs_batch(68)
    o, hf = _run_prefill(p)
    bf = torch.bfloat16
    cu = p.cu_seqlens
    for n in list(range(0, p.N, 7)) + [p.N - 3, p.N - 2, p.N - 1]:
        s, e = int(cu[n]), int(cu[n + 1])
        if e == s:
            continue
        on, hn = kda.chunk_fwd(dev(p.q[s:e], bf), dev(p.k[s:e], bf), dev(p.v[s:e], bf),
                               dev(p.log_alpha[s:e]), dev(p.beta[s:e]), dev(p.h0[n:n + 1]))
        torch.cuda.synchronize()
        assert np.array_equal(host(on), o[s:e]) and np.array_equal(host(hn)[0], hf[n]), n


def test_two_tile_carry_matches_oracle():
    p = _many_pairs_batch(60)
    assert p.N * p.H * 8 > 256
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf)
    rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0, p.cu_seqlens)[1]
    for n in range(p.N):   # every sequence's final state, the empty ones included
        assert rel_fro_err(hf[n], rh[n]) <= TOL[p.io][1], n


def test_two_tile_carry_equals_one_tile_bitwise():
    """Each sequence of the batch run alone (two pairs: one tile per
    workgroup) gives bit-identical outputs and final states: the two-tile
    workgroup does the same arithmetic per tile."""
    p = _many_pairs_batch(61)
    bf = torch.bfloat16
    o_all, hf_all = kda.chunk_fwd(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha),
                                  dev(p.beta), dev(p.h0), dev(p.cu_seqlens, torch.int32))
    torch.cuda.synchronize()
    for n in range(p.N):
        a, b = int(p.cu_seqlens[n]), int(p.cu_seqlens[n + 1])
        o_n, hf_n = kda.chunk_fwd(dev(p.q[a:b], bf), dev(p.k[a:b], bf), dev(p.v[a:b], bf),
                                  dev(p.log_alpha[a:b]), dev(p.beta[a:b]), dev(p.h0[n:n + 1]),
                                  None)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_all[a:b]), n
        assert torch.equal(hf_n[0], hf_all[n]), n


def test_two_tile_carry_single_sequence_many_heads():
    """One sequence with 40 heads (320 one-tile workgroups): the two-tile
    path without the chunk map."""
    p = workloads.make_prefill([333], H=40, seed=62, io="bf16", h0_std=0.05)
    o, hf = _run_prefill(p)
    _check_prefill(p, o, hf, heads=[0, 17, 39])


# -------------------------------------------------- intermediates & layout
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_workspace_intermediates_match_chunkwise_oracle(io):
    """The per-chunk operands the intra-chunk kernel leaves in the workspace
    (W, Qt = Gamma*Q - A_qk W, K', U, Ut = A_qk U, gamma_C) against the fp64
    chunkwise oracle's W, U, A_qk, g for every chunk of two sequences, one of
    them ending in a partial chunk."""
    from oracle import chunkwise
    from tests.kda_testutil import decode_block
    lens = [150, 64]
    H = 2
    p = workloads.make_prefill(lens, H=H, seed=31, io=io, h0_std=0.05)
    dt = io_dtype(io)
    pre = kda.Prefill(dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
                      dev(p.h0), dev(p.cu_seqlens, torch.int32))
    pre.run()
    torch.cuda.synchronize()
    ws = pre.workspace.cpu().numpy().tobytes()
    _, _, parts = chunkwise.chunk_forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0,
                                          p.cu_seqlens, keep_parts=True)
    tol = 1e-4 if io == "f32" else 1.5e-2
    b = 0
    for n, L in enumerate(lens):
        for cidx in range((L + 63) // 64):
            for h in range(H):
                ref = parts[(n, h)][cidx]
                s = ref["start"]
                m = ref["W"].shape[0]
                K = p.k[s:s + m, h].astype(np.float64)
                Q = p.q[s:s + m, h].astype(np.float64)
                g = ref["g"]
                want = dict(W=ref["W"], U=ref["U"],
                            Qt=np.exp(g) * Q - ref["Aqk"] @ ref["W"],
                            Ut=ref["Aqk"] @ ref["U"],
                            Kp=K * np.exp(g[-1][None, :] - g))
                got = decode_block(ws, b + cidx, h, H, len(lens), io)
                for key, val in want.items():
                    full = np.zeros((64, 128))
                    full[:m] = val
                    err = np.abs(got[key] - full).max() / max(np.abs(full).max(), 1e-30)
                    assert err <= tol, (n, cidx, h, key, err)
                gerr = np.abs(got["gC"] - np.exp(g[-1])).max()
                assert gerr <= (1e-6 if io == "f32" else 1e-6), gerr
        b += (L + 63) // 64


# ---------------------------------------------------- call semantics on GPU
def test_h_final_in_place_continuation():
    p = workloads.make_prefill([200, 77], H=3, seed=32, io="bf16", h0_std=0.05)
    bf = torch.bfloat16
    args = [dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha), dev(p.beta)]
    cu = dev(p.cu_seqlens, torch.int32)
    o1, h1 = kda.chunk_fwd(*args, dev(p.h0), cu)
    state = dev(p.h0)
    o2, h2 = kda.chunk_fwd(*args, state, cu, h_final=state)
    torch.cuda.synchronize()
    assert h2.data_ptr() == state.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(h1, state)


def test_split_resume_matches_single_call():
    T, T1 = 333, 129
    p = workloads.make_prefill([T], H=2, seed=33, io="bf16", h0_std=0.05)
    bf = torch.bfloat16

    def run(s, e, h0):
        return kda.chunk_fwd(dev(p.q[s:e], bf), dev(p.k[s:e], bf), dev(p.v[s:e], bf),
                             dev(p.log_alpha[s:e]), dev(p.beta[s:e]), h0)
    o, hf = run(0, T, dev(p.h0))
    oa, ha = run(0, T1, dev(p.h0))
    ob, hb = run(T1, T, ha)
    torch.cuda.synchronize()
    o_split = np.concatenate([host(oa), host(ob)])
    ro, rh = recurrent.forward(p.q, p.k, p.v, p.log_alpha, p.beta, p.h0)
    assert rel_max_err(o_split, ro) <= TOL["bf16"][0]
    assert rel_fro_err(host(hb), rh) <= TOL["bf16"][1]
    assert rel_max_err(o_split, host(o)) <= TOL["bf16"][0]


def test_packed_equals_separate_bitwise():
    lens = [70, 130, 1, 64]
    p = workloads.make_prefill(lens, H=2, seed=34, io="bf16", h0_std=0.05)
    bf = torch.bfloat16
    o, hf = kda.chunk_fwd(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha),
                          dev(p.beta), dev(p.h0), dev(p.cu_seqlens, torch.int32))
    cu = p.cu_seqlens
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = kda.chunk_fwd(dev(p.q[s:e], bf), dev(p.k[s:e], bf), dev(p.v[s:e], bf),
                               dev(p.log_alpha[s:e]), dev(p.beta[s:e]), dev(p.h0[n:n + 1]))
        torch.cuda.synchronize()
        assert torch.equal(on, o[s:e]) and torch.equal(hn[0], hf[n])


@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_identity_padding(path):
    """Tokens with k = 0, v = 0, beta = 0 and log alpha = 0 leave the state
    unchanged: appending 28 of them (and 61 to a second sequence) changes
    neither the final states nor the outputs of the real tokens, bit for
    bit, on either forward path."""
    lens, pads = [100, 3], [28, 61]
    p = workloads.make_prefill(lens, H=2, seed=36, io="bf16", h0_std=0.05)
    parts = {n: [] for n in ("q", "k", "v", "log_alpha", "beta")}
    for n_, (L, P) in enumerate(zip(lens, pads)):
        s0 = int(p.cu_seqlens[n_])
        for name in parts:
            x = getattr(p, name)[s0:s0 + L]
            pad = np.zeros((P,) + x.shape[1:], x.dtype)
            if name == "q":
                pad = p.q[:P].copy()           # any query: its output is not compared
            parts[name].append(np.concatenate([x, pad]))
    padded = {name: np.concatenate(v) for name, v in parts.items()}
    cu_pad = np.concatenate([[0], np.cumsum([L + P for L, P in zip(lens, pads)])]).astype(np.int32)
    bf = torch.bfloat16
    fwd = kda.chunk_fwd if path == "chunk" else kda.recurrent_fwd
    o1, h1 = fwd(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha), dev(p.beta),
                 dev(p.h0), dev(p.cu_seqlens, torch.int32))
    o2, h2 = fwd(dev(padded["q"], bf), dev(padded["k"], bf), dev(padded["v"], bf),
                 dev(padded["log_alpha"]), dev(padded["beta"]), dev(p.h0),
                 dev(cu_pad, torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)
    for n_, L in enumerate(lens):
        a, b = int(p.cu_seqlens[n_]), int(cu_pad[n_])
        assert torch.equal(o1[a:a + L], o2[b:b + L]), n_


def test_decode_steps_match_prefill():
    """64 single-token decode steps equal one prefill over the same tokens."""
    N, H, steps = 4, 2, 64
    S0 = workloads.make_decode_state(N, H, seed=35, std=0.05)
    toks = [workloads.make_decode_step(N, H, seed=35, step=s, io="bf16") for s in range(steps)]
    bf = torch.bfloat16
    S = dev(S0)
    outs = []
    for d in toks:
        outs.append(host(kda.decode_step(dev(d.q, bf), dev(d.k, bf), dev(d.v, bf),
                                         dev(d.log_alpha), dev(d.beta), S)))
    # the same tokens as N sequences of length 64, packed sequence-major
    def pack(name):
        return np.stack([getattr(d, name) for d in toks], axis=1).reshape(
            (N * steps,) + getattr(toks[0], name).shape[1:])
    cu = np.arange(N + 1, dtype=np.int32) * steps
    o, hf = kda.chunk_fwd(dev(pack("q"), bf), dev(pack("k"), bf), dev(pack("v"), bf),
                          dev(pack("log_alpha")), dev(pack("beta")), dev(S0),
                          dev(cu, torch.int32))
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=1).reshape(N * steps, H, 128)
    assert rel_max_err(o_dec, host(o)) <= 2e-2
    assert rel_fro_err(host(S), host(hf)) <= 1e-2


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_exact_recall(io):
    """|k| = 1, beta = 1, q = k: each token reads back its own value."""
    p = workloads.make_prefill([190], H=2, seed=36, io=io, h0_std=0.05)
    p.beta[:] = 1.0
    dt = io_dtype(io)
    o, _ = kda.chunk_fwd(dev(p.k, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha),
                         dev(p.beta), dev(p.h0))
    torch.cuda.synchronize()
    ro, _ = recurrent.forward(p.k, p.k, p.v, p.log_alpha, p.beta, p.h0)
    tol = TOL[io][0]
    assert rel_max_err(host(o), ro) <= tol
    # the oracle reproduces v up to the rounding of k to the I/O dtype
    assert rel_max_err(host(o), p.v.astype(np.float64)) <= (1e-3 if io == "f32" else 3e-2)


def test_binding_reports_rejected_arguments():
    """The binding turns a rejected call into KDAError with the ABI status:
    a q view starting 8 bytes into its allocation (misaligned), and an
    output overlapping an input."""
    p = workloads.make_prefill([100], H=2, seed=44, io="bf16", h0_std=0.05)
    bf = torch.bfloat16
    q_big = torch.zeros(p.q.size + 8, dtype=bf, device="cuda")
    q_off = q_big[4:4 + p.q.size].view(p.q.shape)           # 8 bytes in
    q_off.copy_(dev(p.q, bf))
    args = (dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha), dev(p.beta))
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd(q_off, *args, dev(p.h0))
    assert e.value.status == kda.KDA_ERR_ALIGN
    q = dev(p.q, bf)
    with pytest.raises(kda.KDAError) as e:
        kda.chunk_fwd(q, *args, dev(p.h0), o=q)
    assert e.value.status == kda.KDA_ERR_ALIAS


def test_zero_tokens_keep_initial_state():
    H = 2
    h0 = workloads.make_decode_state(3, H, seed=37, std=0.05)
    e = torch.empty((0, H, 128), dtype=torch.bfloat16, device="cuda")
    o, hf = kda.chunk_fwd(e, e, e, torch.empty((0, H, 128), device="cuda"),
                          torch.empty((0, H), device="cuda"), dev(h0),
                          dev(np.zeros(4, np.int32), torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(hf, dev(h0))


def test_malformed_cu_seqlens_sets_status():
    """A decreasing cu_seqlens is caught by the chunk map: status word 1, the
    other kernels return without touching memory."""
    p = workloads.make_prefill([100], H=1, seed=38, io="bf16")
    bf = torch.bfloat16
    cu = dev(np.array([0, 60, 20, 100], np.int32), torch.int32)
    pre = kda.Prefill(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha),
                      dev(p.beta), None, cu)
    pre.o.fill_(7.0)
    pre.run()
    torch.cuda.synchronize()
    assert int(pre.workspace[:4].view(torch.int32)[0]) == 1
    assert bool((pre.o == 7.0).all())


def test_malformed_single_sequence_cu_sets_status():
    """One sequence: the full call runs without the chunk-map launch, so the
    two kernels check cu_seqlens themselves; a wrong end offset still gives
    status 1 and leaves o untouched."""
    p = workloads.make_prefill([100], H=1, seed=41, io="bf16")
    bf = torch.bfloat16
    cu = dev(np.array([0, 95], np.int32), torch.int32)
    pre = kda.Prefill(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha),
                      dev(p.beta), None, cu)
    pre.o.fill_(7.0)
    pre.run()
    torch.cuda.synchronize()
    assert int(pre.workspace[:4].view(torch.int32)[0]) == 1
    assert bool((pre.o == 7.0).all())


@pytest.mark.parametrize("cu", [True, False])
def test_single_sequence_phases_equal_full_call(cu):
    """For one sequence the full call skips the chunk map; phase by phase
    (which launches it) gives the same outputs, state and workspace words."""
    p = workloads.make_prefill([333], H=3, seed=42, io="bf16", h0_std=0.05)
    bf = torch.bfloat16
    pre = kda.Prefill(dev(p.q, bf), dev(p.k, bf), dev(p.v, bf), dev(p.log_alpha),
                      dev(p.beta), dev(p.h0), dev(p.cu_seqlens, torch.int32) if cu else None)
    o1, h1 = (x.clone() for x in pre.run())
    torch.cuda.synchronize()
    words1 = pre.workspace[:512].clone()
    pre.workspace[:512].fill_(0xEE)
    for ph in range(3):
        pre.run_phase(ph)
    torch.cuda.synchronize()
    assert torch.equal(pre.o, o1) and torch.equal(pre.h_final, h1)
    w = pre.workspace[:512].view(torch.int32)
    w1 = words1.view(torch.int32)
    assert int(w[0]) == int(w1[0]) == 0                      # status
    assert int(w[64]) == int(w1[64]) == 0                    # chunk_offset[0] at byte 256
    assert int(w[65]) == int(w1[65]) == (333 + 63) // 64     # chunk_offset[1]
    _check_prefill(p, host(o1), host(h1))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_outputs_stay_inside_their_buffers(io):
    """Canaries around o and h_final survive a packed call with ragged tails."""
    lens = [65, 3, 190]
    H = 3
    p = workloads.make_prefill(lens, H=H, seed=39, io=io, h0_std=0.05)
    dt = io_dtype(io)
    T, N, pad = sum(lens), len(lens), 4096
    o_buf = torch.full((T * H * 128 + 2 * pad,), 3.0, dtype=dt, device="cuda")
    h_buf = torch.full((N * H * 128 * 128 + 2 * pad,), 5.0, dtype=torch.float32, device="cuda")
    o = o_buf[pad:pad + T * H * 128].view(T, H, 128)
    hf = h_buf[pad:pad + N * H * 128 * 128].view(N, H, 128, 128)
    kda.chunk_fwd(dev(p.q, dt), dev(p.k, dt), dev(p.v, dt), dev(p.log_alpha), dev(p.beta),
                  dev(p.h0), dev(p.cu_seqlens, torch.int32), o=o, h_final=hf)
    torch.cuda.synchronize()
    assert bool((o_buf[:pad] == 3.0).all()) and bool((o_buf[-pad:] == 3.0).all())
    assert bool((h_buf[:pad] == 5.0).all()) and bool((h_buf[-pad:] == 5.0).all())
    _check_prefill(p, host(o), host(hf))
