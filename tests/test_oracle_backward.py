"""Pins of the float64 gradient oracle (oracle/backward.py).

The gradients autograd computes through the plain PyTorch restatement of the
recurrence are checked against central finite differences of the
independent C oracle: for random directions V, (L(p + hV) - L(p - hV)) / 2h
must equal <dL/dp, V>.  The PyTorch restatement itself must reproduce the C
oracle's forward.
"""
import numpy as np
import pytest
import torch

from oracle import backward, oracle


def _problem(seed, B, T, H, d_in, d_out, n_lr=4, per_seq=False):
    rng = np.random.default_rng(seed)
    m = d_out + 2 * d_in + n_lr
    x = rng.standard_normal((B, T, H, d_in))
    W0 = rng.standard_normal(((B,) if per_seq else ()) + (H, m, d_in)) * d_in ** -0.5 * 1.5
    gy = rng.standard_normal((B, T, H, d_out))
    gW = rng.standard_normal((B, H, m, d_in))
    return x, W0, gy, gW


def _loss(x, W0, flag, gy, gW, n_lr, reset):
    y, WT = oracle.forward(x, W0, flag, n_lr=n_lr, reset_interval=reset)
    return float((y * gy).sum() + (WT * gW).sum())


@pytest.mark.parametrize("flag,n_lr,reset,per_seq", [
    (False, 4, 0, False), (True, 4, 0, False), (False, 1, 0, False), (True, 4, 3, False),
    (False, 4, 0, True)])
def test_torch_forward_matches_c_oracle(flag, n_lr, reset, per_seq):
    x, W0, _, _ = _problem(1, 2, 9, 2, 5, 3, n_lr, per_seq)
    y, WT = oracle.forward(x, W0, flag, n_lr=n_lr, reset_interval=reset)
    yt, WTt = backward.forward_torch(torch.tensor(x), torch.tensor(W0), flag, n_lr, reset)
    np.testing.assert_allclose(yt.numpy(), y, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(WTt.numpy(), WT, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("flag,n_lr,reset,per_seq", [
    (False, 4, 0, False), (True, 4, 0, False), (False, 1, 0, False), (True, 1, 0, False),
    (False, 4, 4, False), (True, 4, 0, True)])
def test_gradients_match_finite_differences(flag, n_lr, reset, per_seq):
    x, W0, gy, gW = _problem(2, 2, 11, 2, 4, 3, n_lr, per_seq)
    dx, dW = backward.grads(x, W0, flag, gy, gW, n_lr, reset)
    rng = np.random.default_rng(3)
    h = 1e-5
    for _ in range(3):
        Vx = rng.standard_normal(x.shape)
        VW = rng.standard_normal(W0.shape)
        fd_x = (_loss(x + h * Vx, W0, flag, gy, gW, n_lr, reset)
                - _loss(x - h * Vx, W0, flag, gy, gW, n_lr, reset)) / (2 * h)
        fd_W = (_loss(x, W0 + h * VW, flag, gy, gW, n_lr, reset)
                - _loss(x, W0 - h * VW, flag, gy, gW, n_lr, reset)) / (2 * h)
        np.testing.assert_allclose((dx * Vx).sum(), fd_x, rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose((dW * VW).sum(), fd_W, rtol=1e-6, atol=1e-8)


def test_gradient_of_frozen_dynamics_is_linear_map():
    # With equal key and query blocks nothing ever moves (q_t = k_t), so
    # y_t = W0[Y] u_t and W_T = W0; the gradient of <gy, y> + <gW, W_T> with
    # respect to W0[Y] is then sum_t gy[t] x_t^T + gW[Y] in closed form,
    # and with respect to x it is W0[Y]^T gy[t].
    x, W0, gy, gW = _problem(4, 1, 6, 1, 4, 3)
    d_in, d_out = 4, 3
    W0[:, d_out + d_in:d_out + 2 * d_in] = W0[:, d_out:d_out + d_in]
    dx, dW = backward.grads(x, W0, False, gy, gW)
    np.testing.assert_allclose(dW[0, :d_out], np.einsum("to,ti->oi", gy[0, :, 0], x[0, :, 0]) + gW[0, 0, :d_out],
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dx[0, :, 0], gy[0, :, 0] @ W0[0, :d_out], rtol=1e-12, atol=1e-12)


def test_reset_every_step_has_closed_form_gradient():
    # With R = 1 every step starts from W0 (SRWM review page Sec. 4.5, read as
    # a return to the initial state), so y_t = W0[Y] x_t and, without a cost
    # on W_T, dL/dW0 = sum_t gy[t] x_t^T in the y rows and 0 elsewhere, and
    # dL/dx_t = W0[Y]^T gy[t].
    x, W0, gy, _ = _problem(5, 2, 7, 2, 4, 3)
    d_out = 3
    dx, dW = backward.grads(x, W0, False, gy, None, 4, 1)
    np.testing.assert_allclose(dW[:, :d_out], np.einsum("btho,bthi->hoi", gy, x), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dW[:, d_out:], 0.0)
    np.testing.assert_allclose(dx, np.einsum("btho,hoi->bthi", gy, W0[:, :d_out]), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("flag,n_lr", [(False, 4), (True, 1)])
def test_reset_gradient_is_sum_over_independent_windows(flag, n_lr):
    # Windows [0,R), [R,2R), ... each start from W0 and never see each other,
    # so the reset run's gradient is the windows' gradients taken as separate
    # runs: dx concatenated over t, dW0 summed; only the last window's final
    # state is W_T.
    R, T = 4, 11
    x, W0, gy, gW = _problem(6, 2, T, 2, 4, 3, n_lr)
    dx, dW = backward.grads(x, W0, flag, gy, gW, n_lr, R)
    dx_w, dW_w = [], np.zeros_like(W0)
    for t0 in range(0, T, R):
        t1 = min(t0 + R, T)
        a, b = backward.grads(x[:, t0:t1], W0, flag, gy[:, t0:t1], gW if t1 == T else None, n_lr)
        dx_w.append(a)
        dW_w += b
    np.testing.assert_allclose(dx, np.concatenate(dx_w, axis=1), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dW, dW_w, rtol=1e-11, atol=1e-12)
