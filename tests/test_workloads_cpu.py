"""The seeded input generators that serve both the oracle and the GPU path:
the same seed gives the same inputs, and the draws follow the recipe (unit
q and k rows, beta in (0, 1), log alpha = log(sigmoid(z)) / 16 or the split
recipe, bf16 values that are bf16-representable, packed lengths inside
their bounds)."""
import numpy as np
import pytest

from gated_delta_rule_50_amd import workloads


def test_same_seed_same_inputs():
    a = workloads.make_prefill([70, 0, 5], H=2, seed=7, io="bf16", h0_std=0.02)
    b = workloads.make_prefill([70, 0, 5], H=2, seed=7, io="bf16", h0_std=0.02)
    c = workloads.make_prefill([70, 0, 5], H=2, seed=8, io="bf16", h0_std=0.02)
    for name in ("q", "k", "v", "log_alpha", "beta", "h0", "cu_seqlens"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert not np.array_equal(a.q, c.q) and not np.array_equal(a.log_alpha, c.log_alpha)
    d1 = workloads.make_decode_step(4, 2, seed=5, step=3)
    d2 = workloads.make_decode_step(4, 2, seed=5, step=3)
    d3 = workloads.make_decode_step(4, 2, seed=5, step=4)
    assert np.array_equal(d1.q, d2.q) and np.array_equal(d1.beta, d2.beta)
    assert not np.array_equal(d1.q, d3.q)
    assert np.array_equal(workloads.make_decode_state(3, 2, seed=9),
                          workloads.make_decode_state(3, 2, seed=9))


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_recipe(io):
    p = workloads.make_prefill([300], H=4, seed=11, io=io)
    for x in (p.q, p.k):
        n = np.linalg.norm(x.astype(np.float64), axis=-1)
        assert np.allclose(n, 1.0, atol=1e-6 if io == "f32" else 8e-3)
    assert (p.beta > 0).all() and (p.beta < 1).all()
    assert (p.log_alpha < 0).all()
    # log(sigmoid(z)) / 16 with z ~ N(0, 1): mean of -softplus(-z) / 16 is about -0.05
    assert -0.06 < p.log_alpha.mean() < -0.04
    if io == "bf16":
        for x in (p.q, p.k, p.v):
            assert np.array_equal(workloads.round_bf16(x), x)
    assert p.h0 is None or not p.h0.any()


def test_split_decay_recipe():
    p = workloads.make_prefill([200], H=2, seed=12, io="bf16", decay="split")
    hi = p.log_alpha[..., 64:]
    assert (hi >= -1.0).all() and (hi <= -0.25).all()
    assert -0.06 < p.log_alpha[..., :64].mean() < -0.04


def test_round_bf16_is_nearest_even():
    x = np.array([1.0 + 2.0 ** -8,            # halfway: even neighbour 1.0
                  1.0 + 3 * 2.0 ** -8,        # halfway: even neighbour 1 + 2^-6
                  1.0 + 2.0 ** -8 + 2.0 ** -20,
                  -1.5,
                  3.0e38], np.float32)                # bf16 spacing there is 2^120:
    # 3.0e38 / 2^120 = 225.7, so the nearest bf16 value is 226 * 2^120
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -1.5, 226 * 2.0 ** 120], np.float32)
    assert np.array_equal(workloads.round_bf16(x), want)


def test_packed_lengths_recipe():
    cfg = workloads.config(3)
    assert cfg.n_seqs == 16 and len(cfg.lengths) == 16
    assert all(512 <= L <= 16384 for L in cfg.lengths)
    assert cfg.lengths == workloads.config(3).lengths      # seeded
    assert workloads.config(1).lengths == (8192,) and workloads.config(4).kind == "decode"


def test_packed_lengths_are_the_first_draw():
    """The packed batch draws its lengths first from the batch's own stream,
    then q (the recipe's draw order): a batch drawn with draw_lengths has the
    q of a stream that skipped exactly those draws."""
    import numpy as np
    spec = (5, 16, 80)
    lengths = workloads.varlen_lengths(77, *spec)
    p = workloads.make_prefill(lengths, 2, seed=77, io="f32", draw_lengths=spec)
    rng = np.random.default_rng(77)
    rng.integers(16, 80, size=5, endpoint=True)
    q0 = rng.standard_normal((sum(lengths), 2, 128), dtype=np.float32)
    q0 = (q0 / np.linalg.norm(q0.astype(np.float64), axis=-1, keepdims=True)).astype(np.float32)
    assert np.allclose(p.q, q0, rtol=0, atol=1e-7)
    with pytest.raises(ValueError):
        workloads.make_prefill((16,) * 5, 2, seed=77, io="f32", draw_lengths=spec)


def test_empty_batch_draws():
    """A batch of empty sequences draws only its initial states."""
    p = workloads.make_prefill([0, 0, 0], 2, seed=608, io="bf16", h0_std=0.05)
    assert p.T == 0 and p.q.shape == (0, 2, 128) and p.h0.shape == (3, 2, 128, 128)
