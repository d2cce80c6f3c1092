"""Property tests of the oracle over random small shapes (hypothesis, seeded
and bounded): the identities the pages fix hold for every shape, not only the
hand-picked ones of tests/test_oracle_pins.py."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)

shapes = st.tuples(st.integers(1, 6), st.integers(1, 6), st.sampled_from([4, 1]), st.booleans(),
                   st.integers(0, 2 ** 31 - 1))


def problem(d_in, d_out, n_lr, T, seed, B=2, H=2, scale=1.0):
    r = np.random.default_rng(seed)
    m = oracle.m_rows(d_in, d_out, n_lr)
    x = r.standard_normal((B, T, H, d_in))
    W0 = r.standard_normal((H, m, d_in)) * scale / np.sqrt(d_in)
    return x, W0


@SETTINGS
@given(shapes, st.integers(1, 12))
def test_continuation_any_split(sh, T):
    # running T1 steps and then T - T1 from W_T1 equals running T steps
    d_in, d_out, n_lr, flag, seed = sh
    x, W0 = problem(d_in, d_out, n_lr, T, seed)
    y, WT = oracle.forward(x, W0, flag, n_lr=n_lr)
    T1 = seed % (T + 1)
    ya, Wa = oracle.forward(x[:, :T1], W0, flag, n_lr=n_lr)
    yb, Wb = oracle.forward(x[:, T1:], Wa, flag, n_lr=n_lr)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(Wb, WT)


@SETTINGS
@given(shapes)
def test_step_delta_identities(sh):
    # after one step, per row i: W_t[i] = W_{t-1}[i] + g_i (v_i - vb_i) kh, so
    # W_t kh = vb + g |kh|^2 (v - vb) and W_t z = W_{t-1} z + g (kh.z)(v - vb)
    d_in, d_out, n_lr, flag, seed = sh
    r = np.random.default_rng(seed)
    m = oracle.m_rows(d_in, d_out, n_lr)
    W = r.standard_normal((m, d_in)) * 2
    s = oracle.step(W, r.standard_normal(d_in) * 2, d_out, flag, n_lr)
    kh, v, vb, g = s["kh"], s["v"], s["vb"], s["g"]
    rate = np.zeros(m, dtype=int) if n_lr == 1 else np.array(
        [0] * d_out + [1] * d_in + [2] * d_in + [3] * 4)
    eta = g[rate]
    np.testing.assert_allclose(s["W"] @ kh, vb + eta * (kh @ kh) * (v - vb), rtol=1e-10, atol=1e-12)
    z = r.standard_normal(d_in)
    np.testing.assert_allclose(s["W"] @ z, W @ z + eta * (kh @ z) * (v - vb), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(kh.sum(), 1.0, rtol=1e-14)
    assert 1.0 / d_in - 1e-15 <= kh @ kh <= 1.0 + 1e-15
    # y_t comes from W_{t-1}
    u = s["u"]
    np.testing.assert_allclose(s["y"], W[:d_out] @ u, rtol=1e-12, atol=1e-13)


@SETTINGS
@given(shapes, st.integers(0, 8))
def test_zero_state_is_a_fixed_point(sh, T):
    d_in, d_out, n_lr, flag, seed = sh
    x, W0 = problem(d_in, d_out, n_lr, T, seed)
    y, WT = oracle.forward(x, np.zeros_like(W0), flag, n_lr=n_lr)
    assert not y.any() and not WT.any()


@SETTINGS
@given(shapes, st.integers(1, 8))
def test_four_equal_rates_equal_one_rate(sh, T):
    # the 4-rate form with four identical rate rows stays so and equals the
    # 1-rate form with that row
    d_in, d_out, _, flag, seed = sh
    x, W1 = problem(d_in, d_out, 1, T, seed)
    W4 = np.concatenate([W1, np.repeat(W1[:, -1:], 3, axis=1)], axis=1)
    y1, WT1 = oracle.forward(x, W1, flag, n_lr=1)
    y4, WT4 = oracle.forward(x, W4, flag, n_lr=4)
    np.testing.assert_allclose(y4, y1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(WT4[:, :, :-3], WT1, rtol=1e-11, atol=1e-13)
    for c in range(1, 4):
        np.testing.assert_array_equal(WT4[:, :, -4 + c], WT4[:, :, -4])


@SETTINGS
@given(shapes, st.integers(1, 8))
def test_heads_and_sequences_independent(sh, T):
    d_in, d_out, n_lr, flag, seed = sh
    x, W0 = problem(d_in, d_out, n_lr, T, seed, B=3, H=2)
    y, WT = oracle.forward(x, W0, flag, n_lr=n_lr)
    perm = [2, 0, 1]
    yp, WTp = oracle.forward(x[perm], W0, flag, n_lr=n_lr)
    np.testing.assert_array_equal(yp, y[perm])
    np.testing.assert_array_equal(WTp, WT[perm])
    yh, WTh = oracle.forward(x[:, :, 1:], W0[1:], flag, n_lr=n_lr)
    np.testing.assert_array_equal(yh, y[:, :, 1:])
    np.testing.assert_array_equal(WTh, WT[:, 1:])
