"""Float64 gradient oracle of the SRWM recurrence (plain PyTorch CPU ops).

TEST INFRASTRUCTURE ONLY.  Only tests/ and bench.py's cpu_baseline leg may
import this module; the product path never does.

The pages train the initial matrix W0 (and every other parameter) by
backpropagation through the unrolled self-modification ([ACL] after Eq. (6):
"memory-efficient" BPTT; [SRWM] Sec. 2.5).  This module states the forward
pass once more, as a plain step-by-step PyTorch program in float64 on the CPU
(one batched matrix product per formula, the steps in the order of [ACL]
Eq. (1)-(5)), and lets autograd differentiate it.  The result is pinned to
central finite differences of the independent C oracle (oracle/srwm_oracle.c)
in tests/test_oracle_backward.py.

Loss convention: L = sum_t <gy[t], y_t> + <gW, W_T>; the gradients returned are
dL/dx and dL/dW0 (dW0 has W0's shape: per head when W0 is shared over the
batch, per unit when W0 is [B,H,m,d]).
"""
from __future__ import annotations

import numpy as np
import torch


def forward_torch(x: torch.Tensor, W0: torch.Tensor, apply_input_softmax: bool, n_lr: int = 4,
                  reset_interval: int = 0):
    """x [B,T,H,d_in], W0 [H,m,d_in] or [B,H,m,d_in] (float64) -> (y, W_T)."""
    B, T, H, d_in = x.shape
    m = W0.shape[-2]
    d_out = m - 2 * d_in - n_lr
    W_init = W0.expand(B, H, m, d_in) if W0.dim() == 3 else W0
    W = W_init
    # learning-rate index of every row: its block (y, k, q, beta) or 0
    if n_lr == 4:
        rate = torch.tensor([0] * d_out + [1] * d_in + [2] * d_in + [3] * 4)
    else:
        rate = torch.zeros(m, dtype=torch.long)
    ys = []
    for t in range(T):
        if reset_interval > 0 and t > 0 and t % reset_interval == 0:
            W = W_init
        u = x[:, t]                                           # [B,H,d_in]
        if apply_input_softmax:
            u = torch.softmax(u, dim=-1)
        z = torch.matmul(W, u.unsqueeze(-1)).squeeze(-1)      # Eq. (1), [B,H,m]
        ys.append(z[..., :d_out])                             # from W_{t-1}
        kh = torch.softmax(z[..., d_out:d_out + d_in], dim=-1)
        qh = torch.softmax(z[..., d_out + d_in:d_out + 2 * d_in], dim=-1)
        g = torch.sigmoid(z[..., m - n_lr:])                  # [B,H,n_lr]
        v = torch.matmul(W, qh.unsqueeze(-1)).squeeze(-1)     # Eq. (2)
        vb = torch.matmul(W, kh.unsqueeze(-1)).squeeze(-1)
        a = g[..., rate] * (v - vb)                           # Eq. (5), per row block
        W = W + a.unsqueeze(-1) * kh.unsqueeze(-2)            # Eq. (3), rank one
    y = torch.stack(ys, dim=1) if T > 0 else x.new_zeros((B, 0, H, d_out))
    return y, W


def grads(x, W0, apply_input_softmax: bool, gy, gW=None, n_lr: int = 4, reset_interval: int = 0):
    """Return (dL/dx, dL/dW0) as float64 numpy arrays."""
    xt = torch.tensor(np.asarray(x, np.float64), requires_grad=True)
    Wt = torch.tensor(np.asarray(W0, np.float64), requires_grad=True)
    y, WT = forward_torch(xt, Wt, apply_input_softmax, n_lr, reset_interval)
    L = (y * torch.tensor(np.asarray(gy, np.float64))).sum()
    if gW is not None:
        L = L + (WT * torch.tensor(np.asarray(gW, np.float64))).sum()
    dx, dW = torch.autograd.grad(L, [xt, Wt], allow_unused=True)
    dx = np.zeros_like(np.asarray(x, np.float64)) if dx is None else dx.numpy()
    dW = np.zeros_like(np.asarray(W0, np.float64)) if dW is None else dW.numpy()
    return dx, dW
