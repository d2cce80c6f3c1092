"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each test names the passage (page title + section / equation) or the piece of
mathematics it rests on.  Pages:
  [ACL]  "Metalearning Continual Learning Algorithms -- part 2/5": Sec. 2.3
         Eq. (1)-(3) and the "4-learning-rate version" paragraph, Eq. (4)-(5).
  [SRWM] review page "SRWM: 让权重矩阵学习修改自身" of "A Modern Self-Referential
         Weight Matrix That Learns to Modify Itself": Sec. 2.2-2.5.
"""
import json
import os

import mpmath
import numpy as np
import pytest

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(rng, B, T, H, d_in, d_out, w_std=None):
    m = oracle.m_rows(d_in, d_out)
    x = rng.standard_normal((B, T, H, d_in))
    W0 = rng.standard_normal((H, m, d_in)) * (w_std if w_std else d_in ** -0.5)
    return x, W0


def _blocks(d_in, d_out):
    m = oracle.m_rows(d_in, d_out)
    return [slice(0, d_out), slice(d_out, d_out + d_in), slice(d_out + d_in, d_out + 2 * d_in),
            slice(m - 4, m)]


# --------------------------------------------------------------------------
# P1. [SRWM] Sec. 2.3 worked example, stored under tests/golden with its source.
def test_worked_example_given_addresses():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    W, v, vb = oracle.delta_update(ex["W"], ex["key_address"], ex["query_address"], ex["eta"])
    assert vb[0] == ex["old_value"]
    assert v[0] == ex["target_value"]
    np.testing.assert_array_equal(W, np.array(ex["expected_W"]))


# P2. The same example embedded in the full recurrence: the model must itself
# produce key ~ e1, query ~ e2 and gate 0.5 from W0 and u_1 = e1.  The output
# at step 1 comes from W_0 ([SRWM] Sec. 2.2), the one at step 2 from W_1.
@pytest.mark.parametrize("d_in,d_out", [(2, 1), (8, 8), (5, 3)])
def test_worked_example_in_recurrence(d_in, d_out):
    rng = np.random.default_rng(11)
    m = oracle.m_rows(d_in, d_out)
    L = 20.0
    W0 = rng.standard_normal((1, m, d_in)) * 0.3
    K, Q = d_out, d_out + d_in
    W0[0, :, 0] = 0.0
    W0[0, 0, :2] = [1.0, 3.0]
    W0[0, K:K + d_in, 0] = -L
    W0[0, K, 0] = L                 # key logits: large at address 1
    W0[0, Q:Q + d_in, 0] = -L
    W0[0, Q + 1, 0] = L             # query logits: large at address 2
    W0[0, m - 4:, 0] = 0.0          # all four gates sigmoid(0) = 0.5
    x = np.zeros((1, 2, 1, d_in))
    x[0, :, 0, 0] = 1.0             # u_1 = u_2 = e1
    y, WT = oracle.forward(x, W0, apply_input_softmax=False)
    assert y[0, 0, 0, 0] == 1.0
    np.testing.assert_allclose(y[0, 1, 0, 0], 2.0, rtol=0, atol=1e-12)
    # after step 1 the first y-row reads [2, 3] (step 2 moves it again)
    one = oracle.step(W0[0], x[0, 0, 0], d_out, False)
    np.testing.assert_allclose(one["W"][0, :2], [2.0, 3.0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(one["g"], [0.5] * 4, rtol=0, atol=0)


# P3. [SRWM] Sec. 2.5: an all-zero initial matrix never moves.
@pytest.mark.parametrize("flag", [False, True])
def test_zero_matrix_is_fixed_point(flag):
    rng = np.random.default_rng(3)
    x, _ = _rand_problem(rng, 2, 9, 3, 6, 4)
    W0 = np.zeros((3, oracle.m_rows(6, 4), 6))
    y, WT = oracle.forward(x, W0, flag)
    assert not np.any(y) and not np.any(WT)


# P4. [SRWM] Sec. 2.3 reread identity and associative interference,
# re-derived from [ACL] Eq. (3)/(5) because the page's display formulas were
# lost: per block X, W_t^X kh = vb^X + g_X |kh|^2 (v^X - vb^X) and for any z,
# W_t^X z = W_{t-1}^X z + g_X (kh . z)(v^X - vb^X).  Also the product form
# W_t^X = W_{t-1}^X (I + g_X (qh - kh) kh^T) that follows from
# v - vb = W (qh - kh).  Right-hand sides use numpy products only.
@pytest.mark.parametrize("flag", [False, True])
def test_delta_rule_identities(flag):
    rng = np.random.default_rng(4)
    d_in, d_out = 7, 5
    m = oracle.m_rows(d_in, d_out)
    W = rng.standard_normal((m, d_in)) * 0.8
    for t in range(6):
        xt = rng.standard_normal(d_in) * 2
        r = oracle.step(W, xt, d_out, flag)
        Wn, kh, qh, g, v, vb = r["W"], r["kh"], r["qh"], r["g"], r["v"], r["vb"]
        np.testing.assert_allclose(v, W @ qh, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(vb, W @ kh, rtol=1e-13, atol=1e-13)
        zprobe = rng.standard_normal(d_in)
        for X, blk in enumerate(_blocks(d_in, d_out)):
            lhs = Wn[blk] @ kh
            rhs = vb[blk] + g[X] * (kh @ kh) * (v[blk] - vb[blk])
            np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
            lhs = Wn[blk] @ zprobe
            rhs = W[blk] @ zprobe + g[X] * (kh @ zprobe) * (v[blk] - vb[blk])
            np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
            prod = W[blk] @ (np.eye(d_in) + g[X] * np.outer(qh - kh, kh))
            np.testing.assert_allclose(Wn[blk], prod, rtol=1e-12, atol=1e-12)
        # y_t comes from W_{t-1} (before the update)
        np.testing.assert_allclose(r["y"], W[:d_out] @ r["u"], rtol=1e-13, atol=1e-13)
        W = Wn


# P5. [SRWM] Sec. 2.3: normalised addresses are positive, sum to one and
# satisfy 1/d_in <= |phi(k)|^2 <= 1.
@pytest.mark.parametrize("scale", [0.01, 1.0, 30.0])
def test_address_norm_bounds(scale):
    rng = np.random.default_rng(5)
    d_in, d_out = 9, 4
    m = oracle.m_rows(d_in, d_out)
    W = rng.standard_normal((m, d_in)) * scale
    for t in range(5):
        r = oracle.step(W, rng.standard_normal(d_in), d_out, t % 2 == 1)
        for a in (r["kh"], r["qh"]):
            assert np.all(a >= 0)
            np.testing.assert_allclose(a.sum(), 1.0, rtol=0, atol=1e-14)
            n2 = a @ a
            assert 1.0 / d_in - 1e-15 <= n2 <= 1.0 + 1e-15
        W = r["W"]


# P6. Independent hand expansion at d_in = d_out = 2 (m = 10), three steps,
# in 50-digit arithmetic.  With two addresses, softmax([a, b]) =
# (sigmoid(a - b), sigmoid(b - a)), and writing each row as a sum
# s = w1 + w2 and a difference delta = w1 - w2, one step of the 4-lr rule is
#   z_i    = s_i (u1 + u2)/2 + delta_i (u1 - u2)/2
#   c_i    = g_block(i) * delta_i * (qh1 - kh1)
#   s_i'   = s_i + c_i,   delta_i' = delta_i + c_i (2 kh1 - 1).
# Nothing here calls or mirrors the oracle's loops.
def _sig(a):
    return 1 / (1 + mpmath.exp(-a))


def _brute_force_d2(x, W0, flag):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(float(r[0])) + mpmath.mpf(float(r[1])) for r in W0]
    dl = [mpmath.mpf(float(r[0])) - mpmath.mpf(float(r[1])) for r in W0]
    gate_of_row = [0, 0, 1, 1, 2, 2, 3, 3, 3, 3]
    ys = []
    for x1, x2 in x:
        x1, x2 = mpmath.mpf(float(x1)), mpmath.mpf(float(x2))
        u1, u2 = (_sig(x1 - x2), _sig(x2 - x1)) if flag else (x1, x2)
        z = [s[i] * (u1 + u2) / 2 + dl[i] * (u1 - u2) / 2 for i in range(10)]
        ys.append([z[0], z[1]])
        kh1 = _sig(z[2] - z[3])
        qh1 = _sig(z[4] - z[5])
        g = [_sig(z[6]), _sig(z[7]), _sig(z[8]), _sig(z[9])]
        for i in range(10):
            c = g[gate_of_row[i]] * dl[i] * (qh1 - kh1)
            s[i], dl[i] = s[i] + c, dl[i] + c * (2 * kh1 - 1)
    W = [[(s[i] + dl[i]) / 2, (s[i] - dl[i]) / 2] for i in range(10)]
    return (np.array([[float(v) for v in r] for r in ys]),
            np.array([[float(v) for v in r] for r in W]))


@pytest.mark.parametrize("flag", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_d2_T3(flag, seed):
    rng = np.random.default_rng(100 + seed)
    x = rng.standard_normal((3, 2)) * 1.5
    W0 = rng.standard_normal((10, 2)) * 1.2
    y_bf, W_bf = _brute_force_d2(x, W0, flag)
    y, WT = oracle.forward(x.reshape(1, 3, 1, 2), W0.reshape(1, 10, 2), flag)
    np.testing.assert_allclose(y[0, :, 0], y_bf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(WT[0, 0], W_bf, rtol=1e-12, atol=1e-13)
    # the example must actually move W, or the comparison proves little
    assert np.abs(W_bf - W0).max() > 1e-3


# P7. Constant rows are fixed points (a row c*1 reads c at any probability
# vector, so v_i = vb_i).  Setting the logit row of one gate to -50 with the
# input softmax on makes that gate sigmoid(-50) ~ 2e-22, which freezes
# exactly the block that the 4-lr paragraph of [ACL] assigns to it
# (order y, k, q, beta) while the others keep moving.
@pytest.mark.parametrize("gate", [0, 1, 2, 3])
def test_gate_to_block_assignment(gate):
    rng = np.random.default_rng(7)
    d_in, d_out, T = 6, 5, 12
    m = oracle.m_rows(d_in, d_out)
    x, W0 = _rand_problem(rng, 1, T, 1, d_in, d_out, w_std=1.5)
    W0[0, m - 4 + gate, :] = -50.0
    y, WT = oracle.forward(x, W0, apply_input_softmax=True)
    blocks = _blocks(d_in, d_out)
    for X, blk in enumerate(blocks):
        change = np.abs(WT[0, 0, blk] - W0[0, blk]).max() / np.abs(W0[0, blk]).max()
        if X == gate:
            assert change < 1e-14, (X, change)
        elif X != 3 or gate != 3:
            assert change > 1e-6, (X, change)
    # the constant row itself only moves by rounding (c * sum(qh) vs c * sum(kh))
    np.testing.assert_allclose(WT[0, 0, m - 4 + gate], W0[0, m - 4 + gate], rtol=1e-13)


# P7b. Without the input softmax a constant y-row c*1 outputs c * sum_j x_j.
def test_constant_output_row_closed_form():
    rng = np.random.default_rng(8)
    d_in, d_out, T = 5, 4, 10
    x, W0 = _rand_problem(rng, 1, T, 1, d_in, d_out)
    W0[0, 2, :] = 0.75
    y, WT = oracle.forward(x, W0, apply_input_softmax=False)
    np.testing.assert_allclose(y[0, :, 0, 2], 0.75 * x[0, :, 0, :].sum(-1), rtol=1e-13, atol=1e-13)
    assert np.abs(WT[0, 0, :d_out] - W0[0, :d_out]).max() > 1e-6


# P8. Equal key and query blocks give k_t = q_t, so v = vb and W never moves;
# the output is then the fixed linear map W0[Y] x_t.
@pytest.mark.parametrize("flag", [False, True])
def test_equal_key_query_blocks_freeze(flag):
    rng = np.random.default_rng(9)
    d_in, d_out, T = 6, 3, 8
    x, W0 = _rand_problem(rng, 2, T, 2, d_in, d_out)
    W0[:, d_out + d_in:d_out + 2 * d_in] = W0[:, d_out:d_out + d_in]
    y, WT = oracle.forward(x, W0, flag)
    np.testing.assert_array_equal(WT, np.broadcast_to(W0, WT.shape))
    u = x
    if flag:
        e = np.exp(x - x.max(-1, keepdims=True))
        u = e / e.sum(-1, keepdims=True)
    ref = np.einsum("hoi,bthi->btho", W0[:, :d_out], u)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


# P9. d_in = 1: softmax of one entry is 1, so v = vb and W is constant.
def test_single_input_width_freezes():
    rng = np.random.default_rng(10)
    x, W0 = _rand_problem(rng, 1, 6, 1, 1, 3)
    y, WT = oracle.forward(x, W0, False)
    np.testing.assert_array_equal(WT[0, 0], W0[0])
    np.testing.assert_allclose(y[0, :, 0, :], x[0, :, 0, :] * W0[0, :3, 0], rtol=1e-14)


# P10. The y block is passive: the k, q, beta blocks never read it, and each
# block evolves by right-multiplication, so y and W_T[Y] are linear in W0[Y]
# with the other blocks held fixed.
@pytest.mark.parametrize("flag", [False, True])
def test_output_block_linearity(flag):
    rng = np.random.default_rng(12)
    d_in, d_out, T = 6, 4, 10
    x, W0 = _rand_problem(rng, 1, T, 1, d_in, d_out)
    A = rng.standard_normal((d_out, d_in))
    Bm = rng.standard_normal((d_out, d_in))
    a, b = 0.7, -1.3

    def run(Y):
        W = W0.copy()
        W[0, :d_out] = Y
        return oracle.forward(x, W, flag)

    yA, WA = run(A)
    yB, WB = run(Bm)
    yC, WC = run(a * A + b * Bm)
    np.testing.assert_allclose(yC, a * yA + b * yB, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(WC[..., :d_out, :], a * WA[..., :d_out, :] + b * WB[..., :d_out, :],
                               rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(WC[..., d_out:, :], WA[..., d_out:, :])


# P11. With the input softmax on, adding a constant to every entry of x_t
# changes nothing (softmax is shift invariant).
def test_input_softmax_shift_invariance():
    rng = np.random.default_rng(13)
    x, W0 = _rand_problem(rng, 2, 12, 3, 8, 8)
    shift = rng.standard_normal((2, 12, 3, 1)) * 5
    y1, W1 = oracle.forward(x, W0, True)
    y2, W2 = oracle.forward(x + shift, W0, True)
    np.testing.assert_allclose(y2, y1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(W2, W1, rtol=1e-11, atol=1e-12)


# P12. Units are independent ([SRWM] Sec. 2.4), and the state is the whole
# memory: running T1 steps, then restarting from W_T1, reproduces the run.
def test_unit_independence_and_continuation():
    rng = np.random.default_rng(14)
    x, W0 = _rand_problem(rng, 4, 20, 2, 6, 6)
    x[2] = x[0]
    y, WT = oracle.forward(x, W0, False)
    np.testing.assert_array_equal(y[2], y[0])
    np.testing.assert_array_equal(WT[2], WT[0])
    perm = [3, 1, 0, 2]
    yp, WTp = oracle.forward(x[perm], W0, False)
    np.testing.assert_array_equal(yp, y[perm])
    np.testing.assert_array_equal(WTp, WT[perm])
    ya, WA = oracle.forward(x[1:2, :7], W0, False)
    yb, WB = oracle.forward(x[1:2, 7:], WA[0], False)
    np.testing.assert_array_equal(np.concatenate([ya, yb], 1), y[1:2])
    np.testing.assert_array_equal(WB, WT[1:2])


def test_zero_length_sequence():
    rng = np.random.default_rng(15)
    x, W0 = _rand_problem(rng, 3, 0, 2, 4, 4)
    y, WT = oracle.forward(x, W0, False)
    assert y.shape == (3, 0, 2, 4)
    np.testing.assert_array_equal(WT, np.broadcast_to(W0, WT.shape))


# ---------------------------------------------------------------------------
# One learning rate ([ACL] Eq. (1)-(3) as first written, m = d_out+2*d_in+1).
def _brute_force_d2_one_rate(x, W0, flag):
    # Same (sum, difference) expansion as above with one gate for all 7 rows.
    mpmath.mp.dps = 50
    s = [mpmath.mpf(float(r[0])) + mpmath.mpf(float(r[1])) for r in W0]
    dl = [mpmath.mpf(float(r[0])) - mpmath.mpf(float(r[1])) for r in W0]
    ys = []
    for x1, x2 in x:
        x1, x2 = mpmath.mpf(float(x1)), mpmath.mpf(float(x2))
        u1, u2 = (_sig(x1 - x2), _sig(x2 - x1)) if flag else (x1, x2)
        z = [s[i] * (u1 + u2) / 2 + dl[i] * (u1 - u2) / 2 for i in range(7)]
        ys.append([z[0], z[1]])
        kh1, qh1, g = _sig(z[2] - z[3]), _sig(z[4] - z[5]), _sig(z[6])
        for i in range(7):
            c = g * dl[i] * (qh1 - kh1)
            s[i], dl[i] = s[i] + c, dl[i] + c * (2 * kh1 - 1)
    W = [[(s[i] + dl[i]) / 2, (s[i] - dl[i]) / 2] for i in range(7)]
    return (np.array([[float(v) for v in r] for r in ys]),
            np.array([[float(v) for v in r] for r in W]))


@pytest.mark.parametrize("flag", [False, True])
def test_one_rate_brute_force_d2(flag):
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 2)) * 1.5
    W0 = rng.standard_normal((7, 2)) * 1.2
    y_bf, W_bf = _brute_force_d2_one_rate(x, W0, flag)
    y, WT = oracle.forward(x.reshape(1, 3, 1, 2), W0.reshape(1, 7, 2), flag, n_lr=1)
    np.testing.assert_allclose(y[0, :, 0], y_bf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(WT[0, 0], W_bf, rtol=1e-12, atol=1e-13)


# Four identical rate rows make the four rates equal at every step (identical
# rows read identical values and get identical updates), which is exactly the
# one-rate recurrence with that row.
@pytest.mark.parametrize("flag", [False, True])
def test_one_rate_equals_four_equal_rates(flag):
    rng = np.random.default_rng(22)
    d_in, d_out = 5, 3
    x, W4 = _rand_problem(rng, 2, 15, 2, d_in, d_out)
    W4[:, -4:] = W4[:, -1:]
    W1 = np.ascontiguousarray(W4[:, :-3])
    y4, T4 = oracle.forward(x, W4, flag)
    y1, T1 = oracle.forward(x, W1, flag, n_lr=1)
    np.testing.assert_array_equal(y4, y1)
    np.testing.assert_array_equal(T4[..., :-3, :], T1)
    for i in range(3):
        np.testing.assert_array_equal(T4[..., -4 + i, :], T4[..., -1, :])


# ---------------------------------------------------------------------------
# Per-sequence initial state and state carry ([SRWM] Sec. 3.3: the state
# persists to the end of the episode across truncation windows).
def test_per_sequence_initial_state():
    rng = np.random.default_rng(23)
    x, W0 = _rand_problem(rng, 3, 10, 2, 6, 4)
    y, WT = oracle.forward(x, W0, False)
    yb, WTb = oracle.forward(x, np.ascontiguousarray(np.broadcast_to(W0, (3,) + W0.shape)), False)
    np.testing.assert_array_equal(yb, y)
    np.testing.assert_array_equal(WTb, WT)
    # continuation of a whole batch from its own final states
    ya, WA = oracle.forward(x[:, :4], W0, False)
    yc, WC = oracle.forward(x[:, 4:], WA, False)
    np.testing.assert_array_equal(np.concatenate([ya, yc], 1), y)
    np.testing.assert_array_equal(WC, WT)
    # different initial states per sequence give different outputs
    W0s = np.ascontiguousarray(np.stack([W0, W0 * 0.5, W0 * 2.0]))
    ys, _ = oracle.forward(x, W0s, False)
    np.testing.assert_array_equal(ys[0], y[0])
    assert np.abs(ys[1] - y[1]).max() > 1e-6


# Reset ablation ([SRWM] Sec. 4.5): resetting every R steps equals independent
# runs of the windows [0,R), [R,2R), ... each from W0.
@pytest.mark.parametrize("flag", [False, True])
def test_reset_interval_is_independent_windows(flag):
    rng = np.random.default_rng(24)
    x, W0 = _rand_problem(rng, 2, 23, 2, 6, 4)
    R = 7
    y, WT = oracle.forward(x, W0, flag, reset_interval=R)
    parts = [oracle.forward(np.ascontiguousarray(x[:, a:a + R]), W0, flag) for a in range(0, 23, R)]
    np.testing.assert_array_equal(y, np.concatenate([p[0] for p in parts], 1))
    np.testing.assert_array_equal(WT, parts[-1][1])
    y0, _ = oracle.forward(x, W0, flag)
    np.testing.assert_array_equal(y[:, :R], y0[:, :R])
    assert np.abs(y[:, R:] - y0[:, R:]).max() > 1e-6
