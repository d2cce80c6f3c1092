"""Pins of the DeltaNet / SR-DeltaNet oracle ([SRWM] Sec. 2.1 and Appendix C.1),
each against something other than the oracle's own loops: closed forms of the
first step and of the d_key = 1 case, the delta-rule identities, exact
linearity, continuation, head structure, and SR-DeltaNet with a frozen SRWM
against DeltaNet with the equivalent slow projection."""
import numpy as np
import pytest

from oracle import oracle

P_OF = oracle.proj_rows


def sig(z):
    return 1.0 / (1.0 + np.exp(-z))


def rng(*s):
    return np.random.default_rng(list(s))


def rand_problem(B, T, H, d_in, d_key, d_v, seed=0, scale=1.0):
    r = rng(seed, 7)
    x = r.standard_normal((B, T, H, d_in))
    P = P_OF(d_key, d_v)
    Wslow = r.standard_normal((H * P, H * d_in)) * scale / np.sqrt(H * d_in)
    return x, Wslow


def test_first_step_from_zero_closed_form():
    # F0 = 0: the read at the key is zero, so F_1 = g v kh^T and the query
    # after the write gives y_1 = g (kh . qh) v.  A query before the write
    # would give 0.
    B, H, d_in, d_key, d_v = 3, 2, 5, 4, 3
    x, Wslow = rand_problem(B, 1, H, d_in, d_key, d_v, seed=1, scale=2.0)
    y, FT = oracle.deltanet_forward(x, Wslow, d_key, d_v)
    P = P_OF(d_key, d_v)
    for b in range(B):
        xt = x[b, 0].reshape(-1)
        for h in range(H):
            p = Wslow[h * P:(h + 1) * P] @ xt
            k, v, q, beta = p[:d_key], p[d_key:d_key + d_v], p[d_key + d_v:2 * d_key + d_v], p[-1]
            kh = np.exp(k - k.max()); kh /= kh.sum()
            qh = np.exp(q - q.max()); qh /= qh.sum()
            np.testing.assert_allclose(y[b, 0, h], sig(beta) * (kh @ qh) * v, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(FT[b, h], sig(beta) * np.outer(v, kh), rtol=1e-12, atol=1e-14)


def test_delta_identities():
    # After the write: F_t kh = vb + g |kh|^2 (v - vb) (the key address moves
    # toward the target), and for any address z: F_t z = F_{t-1} z + g (kh.z)(v - vb).
    r = rng(2, 1)
    for d_key, d_v in [(2, 1), (5, 3), (16, 16)]:
        F = r.standard_normal((d_v, d_key))
        p = r.standard_normal(P_OF(d_key, d_v)) * 2
        s = oracle.fast_step(F, p, d_key, d_v)
        v = p[d_key:d_key + d_v]
        g = s["g"][0]
        kh, qh, vb = s["kh"], s["qh"], s["vb"]
        np.testing.assert_allclose(vb, F @ kh, rtol=1e-12)
        np.testing.assert_allclose(s["F"] @ kh, vb + g * (kh @ kh) * (v - vb), rtol=1e-11, atol=1e-13)
        z = r.standard_normal(d_key)
        np.testing.assert_allclose(s["F"] @ z, F @ z + g * (kh @ z) * (v - vb), rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(s["y"], s["F"] @ qh, rtol=1e-12, atol=1e-14)
        assert 1.0 / d_key - 1e-15 <= kh @ kh <= 1.0 + 1e-15


def test_worked_example_write_then_query():
    # One row [1, 3]; key ~ e1, query ~ e2, target value 3, gate 1/2: the
    # write moves the key's content 1 halfway to 3 -> row [2, 3], and the
    # query after the write reads 3.
    L = 20.0
    F = np.array([[1.0, 3.0]])
    p = np.array([L, -L, 3.0, -L, L, 0.0])  # k (2), v (1), q (2), beta
    s = oracle.fast_step(F, p, 2, 1)
    np.testing.assert_allclose(s["F"], [[2.0, 3.0]], atol=1e-15)
    np.testing.assert_allclose(s["y"], [3.0], atol=1e-15)


def test_scalar_key_is_exponential_smoothing():
    # d_key = 1: phi of a scalar is 1, so F_t = (1 - g_t) F_{t-1} + g_t v_t
    # and y_t = F_t (the query address is 1 too).
    B, T, H, d_in, d_v = 2, 30, 3, 4, 3
    x, Wslow = rand_problem(B, T, H, d_in, 1, d_v, seed=3, scale=3.0)
    F0 = rng(3, 2).standard_normal((B, H, d_v, 1))
    y, FT = oracle.deltanet_forward(x, Wslow, 1, d_v, F0=F0)
    P = P_OF(1, d_v)
    for b in range(B):
        for h in range(H):
            f = F0[b, h, :, 0].copy()
            for t in range(T):
                p = Wslow[h * P:(h + 1) * P] @ x[b, t].reshape(-1)
                g = sig(p[-1])
                f = (1 - g) * f + g * p[1:1 + d_v]
                np.testing.assert_allclose(y[b, t, h], f, rtol=1e-11, atol=1e-13)
            np.testing.assert_allclose(FT[b, h, :, 0], f, rtol=1e-11, atol=1e-13)


def test_linear_in_value_rows():
    # From F0 = 0 the fast matrix is linear in the values: scaling the value
    # rows of the slow projection by c scales y and F_T by c (keys, queries
    # and gates are untouched).
    B, T, H, d_in, d_key, d_v = 2, 25, 2, 6, 5, 4
    x, Wslow = rand_problem(B, T, H, d_in, d_key, d_v, seed=4)
    y1, F1 = oracle.deltanet_forward(x, Wslow, d_key, d_v)
    W2 = Wslow.copy()
    P = P_OF(d_key, d_v)
    for h in range(H):
        W2[h * P + d_key:h * P + d_key + d_v] *= -2.5
    y2, F2 = oracle.deltanet_forward(x, W2, d_key, d_v)
    np.testing.assert_allclose(y2, -2.5 * y1, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(F2, -2.5 * F1, rtol=1e-11, atol=1e-13)


def test_continuation_from_fast_state():
    B, T, H, d_in, d_key, d_v = 2, 40, 2, 4, 4, 4
    x, Wslow = rand_problem(B, T, H, d_in, d_key, d_v, seed=5)
    y, FT = oracle.deltanet_forward(x, Wslow, d_key, d_v)
    ya, Fa = oracle.deltanet_forward(x[:, :17], Wslow, d_key, d_v)
    yb, Fb = oracle.deltanet_forward(x[:, 17:], Wslow, d_key, d_v, F0=Fa)
    np.testing.assert_array_equal(np.concatenate([ya, yb], axis=1), y)
    np.testing.assert_array_equal(Fb, FT)


def test_full_width_projection_couples_heads():
    # The slow projection reads the whole input x_t (all heads): perturbing
    # head 1's input changes head 0's output; with a block-diagonal projection
    # it does not.
    B, T, H, d_in, d_key, d_v = 1, 6, 2, 3, 3, 2
    x, Wslow = rand_problem(B, T, H, d_in, d_key, d_v, seed=6)
    x2 = x.copy()
    x2[:, :, 1] += 0.5
    y1, _ = oracle.deltanet_forward(x, Wslow, d_key, d_v)
    y2, _ = oracle.deltanet_forward(x2, Wslow, d_key, d_v)
    assert np.abs(y1[:, :, 0] - y2[:, :, 0]).max() > 1e-6
    P = P_OF(d_key, d_v)
    Wbd = np.zeros_like(Wslow)
    for h in range(H):
        Wbd[h * P:(h + 1) * P, h * d_in:(h + 1) * d_in] = Wslow[h * P:(h + 1) * P, h * d_in:(h + 1) * d_in]
    y1, _ = oracle.deltanet_forward(x, Wbd, d_key, d_v)
    y2, _ = oracle.deltanet_forward(x2, Wbd, d_key, d_v)
    np.testing.assert_array_equal(y1[:, :, 0], y2[:, :, 0])
    assert np.abs(y1[:, :, 1] - y2[:, :, 1]).max() > 1e-6


@pytest.mark.parametrize("n_lr,flag", [(4, False), (4, True), (1, False)])
def test_srdeltanet_with_frozen_srwm_is_deltanet(n_lr, flag):
    # If the SRWM's key and query blocks are equal it never modifies itself
    # (v = vb), so its output is W0[Y] u_t: SR-DeltaNet then equals DeltaNet
    # whose slow projection is block-diagonal with blocks W0[h][Y] (applied to
    # u_t = x_t, or softmax(x_t) with the input activation).
    B, T, H, d_in, d_key, d_v = 2, 20, 3, 4, 3, 5
    P = P_OF(d_key, d_v)
    m = P + 2 * d_in + n_lr
    r = rng(7, n_lr, int(flag))
    x = r.standard_normal((B, T, H, d_in))
    W0 = r.standard_normal((H, m, d_in)) / np.sqrt(d_in)
    W0[:, P + d_in:P + 2 * d_in] = W0[:, P:P + d_in]
    y, WT, FT = oracle.srdeltanet_forward(x, W0, d_key, d_v, apply_input_softmax=flag, n_lr=n_lr)
    np.testing.assert_array_equal(WT, np.broadcast_to(W0, WT.shape))
    Wbd = np.zeros((H * P, H * d_in))
    for h in range(H):
        Wbd[h * P:(h + 1) * P, h * d_in:(h + 1) * d_in] = W0[h, :P]
    u = x
    if flag:
        u = np.exp(x - x.max(-1, keepdims=True))
        u /= u.sum(-1, keepdims=True)
    y2, F2 = oracle.deltanet_forward(u, Wbd, d_key, d_v)
    np.testing.assert_allclose(y, y2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(FT, F2, rtol=1e-11, atol=1e-13)


def test_srdeltanet_srwm_part_is_the_srwm():
    # The SRWM inside SR-DeltaNet evolves exactly as a stand-alone SRWM with
    # d_out = P on the same input (the fast memory never feeds back).
    B, T, H, d_in, d_key, d_v = 2, 15, 2, 4, 3, 3
    P = P_OF(d_key, d_v)
    m = P + 2 * d_in + 4
    r = rng(8)
    x = r.standard_normal((B, T, H, d_in))
    W0 = r.standard_normal((H, m, d_in)) / np.sqrt(d_in)
    y, WT, FT = oracle.srdeltanet_forward(x, W0, d_key, d_v, apply_input_softmax=True)
    ys, WTs = oracle.forward(x, W0, True)
    np.testing.assert_array_equal(WT, WTs)
    # and the fast memory is DeltaNet's fast step driven by the SRWM's outputs
    for b in range(B):
        for h in range(H):
            F = np.zeros((d_v, d_key))
            for t in range(T):
                s = oracle.fast_step(F, ys[b, t, h], d_key, d_v)
                F = s["F"]
                np.testing.assert_allclose(y[b, t, h], s["y"], rtol=1e-13, atol=1e-15)


def test_float32_drift_is_small():
    # Feasibility of a float32 GPU path at the fp32 tolerance (2e-4 relative L2).
    B, T, H, d_in, d_key, d_v = 2, 512, 4, 16, 16, 16
    x, Wslow = rand_problem(B, T, H, d_in, d_key, d_v, seed=9)
    y64, F64 = oracle.deltanet_forward(x, Wslow, d_key, d_v)
    y32, F32 = oracle.deltanet_forward(x.astype(np.float32), Wslow.astype(np.float32), d_key, d_v, f32=True)
    rel = np.linalg.norm(y32 - y64) / np.linalg.norm(y64)
    assert rel < 2e-5, rel
