"""srwm_backward_noalloc through the C ABI against srwm_backward: the same
dx and batch-summed dW0 (bit for bit, and within the gradient tolerance),
on consecutive calls that reuse the library's scratch array, each smaller
than the one before, so a call that read what an earlier one left behind
would show."""
import ctypes

import numpy as np
import pytest
import torch

from self_referential_weight_amd import _lib
from self_referential_weight_amd.workloads import WORKLOADS, gen_gW, gen_gy, gen_W0, gen_x
from tests._parity import rel_l2

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _inputs(w, reset_interval, with_gW):
    import self_referential_weight_amd as srwm
    dev = torch.device("cuda:0")
    x = torch.from_numpy(gen_x(w)).to(dev)
    if w.io_dtype == "bf16":
        x = x.to(torch.bfloat16)
    W0 = torch.from_numpy(gen_W0(w)).to(dev)
    _, W_T, tape = srwm.forward(x, W0, apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr,
                                reset_interval=reset_interval, save_tape=True)
    gy = torch.from_numpy(gen_gy(w)).to(dev)
    gW = torch.from_numpy(gen_gW(w)).to(dev) if with_gW else None
    return x, W_T, tape, gy, gW


def _args(w, x, W_T, tape, gy, gW, dx, dWi, dW0, reset_interval):
    def p(t):
        return t.data_ptr() if t is not None and t.numel() else None
    return _lib.BackwardArgs(
        x=None, W_T=p(W_T), tape=p(tape.rows), gy=p(gy), gW_T=p(gW), dx=p(dx), dW_init=p(dWi), dW0=p(dW0),
        B=w.B, T=w.T, H=w.H, d_in=w.d_in, d_out=w.d_out, m=w.m,
        io_dtype=_lib.SRWM_IO_BF16 if w.io_dtype == "bf16" else _lib.SRWM_IO_F32,
        apply_input_softmax=int(w.apply_input_softmax), n_lr=w.n_lr,
        stream=torch.cuda.current_stream().cuda_stream, reset_interval=reset_interval,
        window_states=p(tape.window_states))


# Consecutive calls, largest first: the first needs two slices of the scratch
# (48 sequences x 16 heads x 196 x 64 floats is more than 32 MiB), the next
# ones overwrite less of it than the call before wrote.
CASES = [
    (WORKLOADS["rl_d64_bf16"].with_(B=48, T=40), 0, True),
    (WORKLOADS["wide_d128"].with_(B=3, T=21), 0, True),
    (WORKLOADS["fewshot_d64"].with_(B=5, H=3, T=30), 7, False),
    (WORKLOADS["multitask_d16"].with_(B=3, T=33, n_lr=1), 0, False),
]


def test_backward_noalloc_matches_backward():
    lib = _lib.load()
    dev = torch.device("cuda:0")
    scratch_floats = lib.srwm_backward_noalloc_scratch_bytes() // 4
    assert CASES[0][0].B * CASES[0][0].H * CASES[0][0].m * CASES[0][0].d_in > scratch_floats
    for w, R, with_gW in CASES:
        say(f"[no-alloc] {w.name} B={w.B} H={w.H} d={w.d_in} T={w.T} n_lr={w.n_lr} reset={R} gW_T={with_gW}")
        x, W_T, tape, gy, gW = _inputs(w, R, with_gW)
        # the existing entry point, with its caller-provided per-unit buffer
        dx_ref = torch.empty((w.B, w.T, w.H, w.d_in), dtype=torch.float32, device=dev)
        dWi = torch.empty((w.B, w.H, w.m, w.d_in), dtype=torch.float32, device=dev)
        dW0_ref = torch.empty((w.H, w.m, w.d_in), dtype=torch.float32, device=dev)
        rc = lib.srwm_backward(ctypes.byref(_args(w, x, W_T, tape, gy, gW, dx_ref, dWi, dW0_ref, R)))
        assert rc == 0, _lib.strerror(rc)
        # the no-allocation entry point: no dW_init; outputs poisoned first
        dx = torch.full_like(dx_ref, float("nan"))
        dW0 = torch.full_like(dW0_ref, float("nan"))
        rc = lib.srwm_backward_noalloc(ctypes.byref(_args(w, x, W_T, tape, gy, gW, dx, None, dW0, R)))
        assert rc == 0, _lib.strerror(rc)
        torch.cuda.synchronize()
        a, b = dW0.cpu().numpy().astype(np.float64), dW0_ref.cpu().numpy().astype(np.float64)
        assert np.isfinite(a).all() and rel_l2(a, b) <= 1e-4
        assert np.abs(a - b).max() <= 1e-3 * np.abs(b).max()
        assert rel_l2(dx.cpu().numpy().astype(np.float64), dx_ref.cpu().numpy().astype(np.float64)) <= 1e-4
        # same kernels, same slices of one order of summation: the same bits
        assert torch.equal(dx, dx_ref) and torch.equal(dW0, dW0_ref), w.name
