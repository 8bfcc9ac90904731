"""Pins for the fp64 oracles (CPU only).

Each test ties the oracle to something other than itself: hand-worked
examples, closed forms of special cases named on the pages (DeltaNet, Gated
DeltaNet, beta = 0), the exact-recall property of the Householder step, and
structural invariants (linearity, column independence, split/resume,
packing, identity padding, chunk-size invariance). A plausible slip in the
oracle (a dropped decay, decay applied after the correction, readout before
the update, a transposed state, an inclusive relative decay, a missing
diagonal in the intra-chunk mask) fails at least one of them.
"""
import json
from pathlib import Path

import numpy as np
import pytest

from oracle import chunkwise, epilogue, recurrent

GOLDEN = Path(__file__).parent / "golden"


def _inputs(seed, T, H=2, dk=8, dv=8, la_scale=0.3, h0=True, N=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -rng.random((T, H, dk)) * la_scale
    b = rng.random((T, H))
    S0 = rng.standard_normal((N, H, dk, dv)) if h0 else None
    return q, k, v, la, b, S0


def _load(name):
    d = json.loads((GOLDEN / name).read_text())
    arr = {k: (None if d[k] is None else np.array(d[k], dtype=np.float64))
           for k in ("q", "k", "v", "alpha", "beta", "h0", "o", "h_final")}
    arr["log_alpha"] = np.log(arr["alpha"])
    return d, arr


# ---------------------------------------------------------------- P1 golden
@pytest.mark.parametrize("name", ["ex1_decay_then_correct.json", "ex2_two_tokens.json"])
def test_golden_recurrent(name):
    _, a = _load(name)
    o, hf = recurrent.forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"], a["h0"])
    np.testing.assert_allclose(o, a["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hf, a["h_final"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("name", ["ex1_decay_then_correct.json", "ex2_two_tokens.json"])
@pytest.mark.parametrize("chunk", [1, 2, 64])
def test_golden_chunkwise(name, chunk):
    _, a = _load(name)
    o, hf, _ = chunkwise.chunk_forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"],
                                       a["h0"], chunk=chunk)
    np.testing.assert_allclose(o, a["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hf, a["h_final"], rtol=0, atol=1e-14)


def test_golden_chunk_intermediates():
    d, a = _load("ex2_two_tokens.json")
    _, _, parts = chunkwise.chunk_forward(a["q"], a["k"], a["v"], a["log_alpha"], a["beta"],
                                          None, chunk=2, keep_parts=True)
    p = parts[(0, 0)][0]
    for key in ("L", "Ti", "W", "U", "Aqk"):
        np.testing.assert_allclose(p[key], np.array(d["chunk2"][key]), rtol=0, atol=1e-14,
                                   err_msg=key)


# ---------------------------------------------------------- P2 exact recall
def test_exact_recall():
    """|k_t| = 1 and beta_t = 1 make the Householder step (I - k k^T) erase the
    old value along k_t before writing v_t, so S_t^T k_t = v_t exactly. With
    q = k the readout is that lookup."""
    q, k, v, la, b, S0 = _inputs(1, T=50, dk=16, dv=8, la_scale=3.0)
    b[:] = 1.0
    o, _ = recurrent.forward(k, k, v, la, b, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


# --------------------------------------------------- P3 / P4 special cases
def _deltanet(q, k, v, b, S0, alpha_scalar=None):
    """Textbook DeltaNet (intelliparadigm.com article, sec. 2.2) and, with a
    scalar gate, Gated DeltaNet (sec. 2.3), in dense matrix form."""
    T, H, dk = k.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    hf = np.zeros((1, H, dk, dv))
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            kt = k[t, h][:, None]
            A = np.eye(dk) - b[t, h] * (kt @ kt.T)
            if alpha_scalar is not None:
                A = alpha_scalar[t, h] * A
            S = A @ S + b[t, h] * kt @ v[t, h][None, :]
            o[t, h] = S.T @ q[t, h]
        hf[0, h] = S
    return o, hf


def test_deltanet_limit():
    q, k, v, la, b, S0 = _inputs(2, T=40)
    la[:] = 0.0
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    o_ref, hf_ref = _deltanet(q, k, v, b, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hf, hf_ref, rtol=0, atol=1e-12)


def test_gated_deltanet_limit():
    q, k, v, la, b, S0 = _inputs(3, T=40)
    lam = -np.random.default_rng(33).random((40, 2)) * 0.5
    la[:] = lam[:, :, None]
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    o_ref, hf_ref = _deltanet(q, k, v, b, S0, alpha_scalar=np.exp(lam))
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(hf, hf_ref, rtol=0, atol=1e-12)


# ------------------------------------------------ P5 beta = 0 closed form
def test_beta_zero_pure_decay():
    q, k, v, la, b, S0 = _inputs(4, T=30, la_scale=1.0)
    b[:] = 0.0
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    G = np.cumsum(la, axis=0)                                # [T, H, dk]
    for t in range(30):
        St = np.exp(G[t])[:, :, None] * S0[0]                # [H, dk, dv]
        np.testing.assert_allclose(o[t], np.einsum("hcj,hc->hj", St, q[t]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(hf[0], np.exp(G[-1])[:, :, None] * S0[0], rtol=0, atol=1e-12)


# --------------------------------------------- P6 chunkwise == recurrence
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130, 200])
@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunkwise_matches_recurrence(T, chunk):
    q, k, v, la, b, S0 = _inputs(10 + T, T=T, dk=8, dv=4, la_scale=1.5)
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    o2, hf2, _ = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=chunk)
    scale = max(np.abs(o).max(), 1.0)
    assert np.abs(o - o2).max() <= 1e-12 * scale
    assert np.abs(hf - hf2).max() <= 1e-12 * max(np.abs(hf).max(), 1.0)


def test_chunkwise_matches_recurrence_d128():
    q, k, v, la, b, S0 = _inputs(5, T=200, H=1, dk=128, dv=128, la_scale=0.2)
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    o2, hf2, _ = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=64)
    assert np.abs(o - o2).max() <= 1e-12 * np.abs(o).max()
    assert np.abs(hf - hf2).max() <= 1e-12 * np.abs(hf).max()


def test_wy_recursion_matches_ut_transform():
    """W, U from the WY recursions equal the UT-transform forms."""
    q, k, v, la, b, S0 = _inputs(6, T=64, H=1, dk=8, dv=4, la_scale=1.0)
    _, _, parts = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=64, keep_parts=True)
    p = parts[(0, 0)][0]
    w, u = chunkwise.wy_auxiliaries(k[:, 0], v[:, 0], b[:, 0], p["g"])
    np.testing.assert_allclose(p["W"], w, rtol=0, atol=1e-12)
    np.testing.assert_allclose(p["U"], u, rtol=0, atol=1e-12)


def test_wy_state_representation():
    """S_r = P_r S_0 + H_r with P_r = Diag(gamma_r) - sum_i Diag(gamma_{i->r}) k_i w_i^T
    and H_r = sum_i Diag(gamma_{i->r}) k_i u_i^T (review, 'The WY representation
    for P and H'), checked against recurrence states at every r."""
    T, dk, dv = 12, 6, 5
    q, k, v, la, b, S0 = _inputs(7, T=T, H=1, dk=dk, dv=dv, la_scale=1.0)
    g = np.cumsum(la[:, 0], axis=0)
    w, u = chunkwise.wy_auxiliaries(k[:, 0], v[:, 0], b[:, 0], g)
    for r in range(T):
        P = np.diag(np.exp(g[r]))
        Hm = np.zeros((dk, dv))
        for i in range(r + 1):
            dec = np.exp(g[r] - g[i])[:, None]
            P = P - dec * k[i, 0][:, None] @ w[i][None, :]
            Hm = Hm + dec * k[i, 0][:, None] @ u[i][None, :]
        _, S_r = recurrent.forward(q[:r + 1], k[:r + 1], v[:r + 1], la[:r + 1], b[:r + 1], S0)
        np.testing.assert_allclose(P @ S0[0, 0] + Hm, S_r[0, 0], rtol=0, atol=1e-12)


# ------------------------------------------------------ P7 linearity
def test_linearity_in_v_and_h0():
    q, k, v1, la, b, A = _inputs(8, T=70)
    _, _, v2, _, _, B = _inputs(9, T=70)
    o1, h1 = recurrent.forward(q, k, v1, la, b, A)
    o2, h2 = recurrent.forward(q, k, v2, la, b, B)
    o3, h3 = recurrent.forward(q, k, v1 + 2 * v2, la, b, A + 2 * B)
    np.testing.assert_allclose(o3, o1 + 2 * o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(h3, h1 + 2 * h2, rtol=0, atol=1e-12)


# ----------------------------------------------- P8 column independence
def test_column_independence():
    q, k, v, la, b, S0 = _inputs(10, T=50, dv=8)
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    v2, S2 = v.copy(), S0.copy()
    v2[:, :, 3] += 1.0
    S2[..., 3] -= 2.0
    o2, hf2 = recurrent.forward(q, k, v2, la, b, S2)
    keep = [j for j in range(8) if j != 3]
    assert np.array_equal(o[..., keep], o2[..., keep])
    assert np.array_equal(hf[..., keep], hf2[..., keep])
    assert not np.allclose(o[..., 3], o2[..., 3])


# ---------------------------------------------------- P9 split / resume
def test_split_resume_bitwise():
    q, k, v, la, b, S0 = _inputs(11, T=90)
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    oa, ha = recurrent.forward(q[:37], k[:37], v[:37], la[:37], b[:37], S0)
    ob, hb = recurrent.forward(q[37:], k[37:], v[37:], la[37:], b[37:], ha)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(hb, hf)


# -------------------------------------------------------- P10 packing
def test_packing_bitwise():
    lens = [5, 0, 17, 64, 1]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q, k, v, la, b, S0 = _inputs(12, T=T, N=len(lens))
    o, hf = recurrent.forward(q, k, v, la, b, S0, cu_seqlens=cu)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        on, hn = recurrent.forward(q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], S0[n:n + 1])
        assert np.array_equal(o[s:e], on)
        assert np.array_equal(hf[n], hn[0])
    assert np.array_equal(hf[1], S0[1])  # empty sequence keeps h0


# ----------------------------------------------- P11 identity padding
def test_identity_tokens_leave_state_unchanged():
    q, k, v, la, b, S0 = _inputs(13, T=20)
    _, hf = recurrent.forward(q, k, v, la, b, S0)
    pad = 7
    rng = np.random.default_rng(5)
    qp = np.concatenate([q, rng.standard_normal((pad, 2, 8))])
    kp = np.concatenate([k, np.zeros((pad, 2, 8))])
    vp = np.concatenate([v, rng.standard_normal((pad, 2, 8))])
    lap = np.concatenate([la, np.zeros((pad, 2, 8))])
    bp = np.concatenate([b, np.zeros((pad, 2))])
    _, hfp = recurrent.forward(qp, kp, vp, lap, bp, S0)
    assert np.array_equal(hf, hfp)


# -------------------------------------------- P12 chunk-size invariance
def test_chunk_size_invariance():
    q, k, v, la, b, S0 = _inputs(14, T=150, la_scale=2.0)
    ref = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=64)
    for C in (1, 3, 16, 150):
        o, hf, _ = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=C)
        assert np.abs(o - ref[0]).max() <= 1e-12 * np.abs(o).max()
        assert np.abs(hf - ref[1]).max() <= 1e-12 * np.abs(hf).max()


def test_strong_decay_no_overflow():
    """Decays far below exp(-88) per chunk (fp32's range) stay finite and
    match the recurrence: no 1/Gamma is ever formed."""
    q, k, v, la, b, S0 = _inputs(15, T=130, la_scale=1.0)
    la[:, :, :4] = -20.0
    o, hf = recurrent.forward(q, k, v, la, b, S0)
    o2, hf2, _ = chunkwise.chunk_forward(q, k, v, la, b, S0, chunk=64)
    assert np.isfinite(o2).all() and np.isfinite(hf2).all()
    assert np.abs(o - o2).max() <= 1e-12 * np.abs(o).max()


# ----------------------------------------------------- decode = 1 token
def test_decode_step_is_one_token_recurrence():
    N, H, d = 3, 2, 8
    rng = np.random.default_rng(16)
    q, k, v = (rng.standard_normal((N, H, d)) for _ in range(3))
    la = -rng.random((N, H, d))
    b = rng.random((N, H))
    S = rng.standard_normal((N, H, d, d))
    o, S1 = recurrent.decode_step(q, k, v, la, b, S)
    for n in range(N):
        on, hn = recurrent.forward(q[n:n + 1], k[n:n + 1], v[n:n + 1], la[n:n + 1],
                                   b[n:n + 1], S[n:n + 1])
        assert np.array_equal(o[n], on[0])
        assert np.array_equal(S1[n], hn[0])


# --------------------------------------------------------- L2 normalisation
def test_l2norm_worked_examples():
    """(3, 4) has length 5; a zero vector stays zero (the epsilon only guards
    the division); each vector along the last axis is scaled on its own."""
    x = np.array([[3.0, 4.0], [0.0, 0.0], [-1e-3, 0.0]])
    y = recurrent.l2norm(x)
    np.testing.assert_allclose(y[0], [0.6, 0.8], rtol=0, atol=1e-7)
    assert np.all(y[1] == 0.0)
    np.testing.assert_allclose(y[2], [-1e-3 / np.sqrt(1e-6 + 1e-6), 0.0], rtol=1e-14)


def test_l2norm_unit_length_and_scale_invariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 3, 128))
    y = recurrent.l2norm(x)
    n2 = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.sqrt(n2 / (n2 + 1e-6)),
                               rtol=1e-14)
    np.testing.assert_allclose(recurrent.l2norm(7.5 * x), y, rtol=0, atol=1e-8)
    # the direction is kept: y is a positive multiple of x
    ratio = y / x
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[..., :1], ratio.shape), rtol=1e-13)
    assert np.all(ratio > 0)


def test_l2norm_feeds_exact_recall():
    """Keys normalised by l2norm (up to the epsilon) satisfy the exact-recall
    property of the Householder step: with beta = 1, S_t^T k_t = v_t."""
    q, k, v, la, b, S0 = _inputs(5, T=40, dk=16, dv=8, la_scale=2.0)
    kn = recurrent.l2norm(5.0 * np.random.default_rng(5).standard_normal(k.shape))
    b[:] = 1.0
    o, _ = recurrent.forward(kn, kn, v, la, b, S0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-5)


# ----------------------------------------------------- RMSNorm x sigmoid gate
def test_sigmoid_closed_forms():
    """sigmoid(0) = 1/2, sigmoid(log 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1,
    and no overflow far from zero."""
    assert epilogue.sigmoid(0.0) == 0.5
    np.testing.assert_allclose(epilogue.sigmoid(np.log(3.0)), 0.75, rtol=1e-15)
    x = np.linspace(-30, 30, 121)
    np.testing.assert_allclose(epilogue.sigmoid(x) + epilogue.sigmoid(-x), 1.0, rtol=1e-15)
    big = epilogue.sigmoid(np.array([-800.0, 800.0]))
    assert big[0] == 0.0 and big[1] == 1.0


def test_rmsnorm_gate_worked_example():
    """o = (3, 4): mean square 12.5, so RMSNorm(o) = o / sqrt(12.5); gate 0
    halves it; weight (1, 2) scales the channels."""
    y = epilogue.rmsnorm_gate(np.array([3.0, 4.0]), np.array([0.0, 0.0]),
                              np.array([1.0, 2.0]), eps=0.0)
    np.testing.assert_allclose(y, [0.5 * 3 / np.sqrt(12.5), 0.5 * 2 * 4 / np.sqrt(12.5)],
                               rtol=1e-15)
    # eps enters under the root: o = (1, 1), eps = 3 gives 1 / 2
    y = epilogue.rmsnorm_gate(np.ones(2), np.full(2, 800.0), None, eps=3.0)
    np.testing.assert_allclose(y, [0.5, 0.5], rtol=1e-15)


def test_rmsnorm_gate_invariants():
    """Per row: unit RMS after the norm (open gate, unit weight), invariance
    to scaling o, rows normalised independently, gate applied elementwise."""
    rng = np.random.default_rng(12)
    o = rng.standard_normal((6, 4, 128)) * rng.uniform(0.1, 10, (6, 4, 1))
    g = rng.standard_normal((6, 4, 128))
    y_open = epilogue.rmsnorm_gate(o, np.full_like(o, 800.0), None, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y_open ** 2, axis=-1)), 1.0, rtol=1e-13)
    y = epilogue.rmsnorm_gate(o, g, None, eps=0.0)
    np.testing.assert_allclose(epilogue.rmsnorm_gate(5.0 * o, g, None, eps=0.0), y, rtol=1e-13)
    o2 = o.copy()
    o2[0, 0] *= 3.0                      # one row changes, the others do not
    y2 = epilogue.rmsnorm_gate(o2, g, None, eps=0.0)
    np.testing.assert_array_equal(y2[1:], y[1:])
    np.testing.assert_array_equal(y2[0, 1:], y[0, 1:])
    np.testing.assert_allclose(y / y_open, epilogue.sigmoid(g), rtol=1e-13)
