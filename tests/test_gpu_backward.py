"""GPU backward pass (through the C ABI) against the float64 gradient oracle
(oracle/backward.py: the recurrence differentiated by autograd in float64,
itself pinned to finite differences of the C oracle).  The loss is
L = sum_t <gy[t], y_t> + <gW_T, W_T>; tolerances in tests/_parity.py."""
import numpy as np
import pytest

from oracle import backward as oracle_bwd
from oracle import oracle
from self_referential_weight_amd.workloads import (WORKLOADS, Workload, gen_gW, gen_gy, gen_W0, gen_x,
                                                   round_to_bf16)
from tests._parity import check_grad, check_state, check_y, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _srwm():
    import self_referential_weight_amd as srwm
    return srwm


def dev():
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def to_dev(a, io_dtype="f32"):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t.to(torch.bfloat16) if io_dtype == "bf16" else t


def gpu_grads(w, x, W0, gy, gW, flag, shared=True, variant=-1, reset_interval=0):
    srwm = _srwm()
    xd = to_dev(x, w.io_dtype)
    y, WT, tape = srwm.forward(xd, to_dev(W0), apply_input_softmax=flag, n_lr=w.n_lr, save_tape=True,
                               variant=variant, reset_interval=reset_interval)
    dx, dW = srwm.backward(xd, WT, tape, to_dev(gy), None if gW is None else to_dev(gW),
                           apply_input_softmax=flag, n_lr=w.n_lr, shared_W0=shared)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), WT.cpu().numpy(), dx.cpu().numpy(), dW.cpu().numpy()


SMALL = {
    "tiny_d8": dict(B=3, H=2, T=40),
    "multitask_d16": dict(),                  # the workload as is: B=4, H=4, T=256
    "fewshot_d64": dict(B=3, H=3, T=200),
    "rl_d64_bf16": dict(B=2, H=3, T=157),
    "wide_d128": dict(B=2, H=2, T=61),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("n_lr", [4, 1])
@pytest.mark.parametrize("flag", [False, True])
@pytest.mark.parametrize("with_gW", [False, True])
def test_backward_parity(name, n_lr, flag, with_gW):
    w = WORKLOADS[name].with_(n_lr=n_lr, **SMALL[name])
    say(f"[bwd] {name} B={w.B} H={w.H} T={w.T} n_lr={n_lr} softmax={flag} gW={with_gW}")
    x, W0, gy = gen_x(w), gen_W0(w), gen_gy(w)
    gW = gen_gW(w) if with_gW else None
    y, WT, dx, dW0 = gpu_grads(w, x, W0, gy, gW, flag)
    y_ref, WT_ref = oracle.forward(x, W0, flag, n_lr=n_lr)
    check_y(y, y_ref, w.io_dtype, "taped forward")
    check_state(WT, WT_ref, "taped forward")
    dx_ref, dW0_ref = oracle_bwd.grads(x, W0, flag, gy, gW, n_lr=n_lr)
    rx = check_grad(dx, dx_ref, "dx")
    rw = check_grad(dW0, dW0_ref, "dW0")
    say(f"[bwd] relL2 dx={rx:.2e} dW0={rw:.2e}")


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_per_sequence_initial_state(name):
    # W0 given per sequence: the backward's per-unit gradient is the gradient
    # of that W0 (no sum over the batch).
    w = WORKLOADS[name].with_(**SMALL[name])
    flag = w.apply_input_softmax
    x, gy, gW = gen_x(w), gen_gy(w), gen_gW(w)
    rng = np.random.default_rng([w.seed, 9])
    W0 = (rng.standard_normal((w.B, w.H, w.m, w.d_in)) * w.w0_std).astype(np.float32)
    _, _, dx, dWi = gpu_grads(w, x, W0, gy, gW, flag, shared=False)
    dx_ref, dWi_ref = oracle_bwd.grads(x, W0, flag, gy, gW, n_lr=w.n_lr)
    assert dWi.shape == W0.shape
    check_grad(dx, dx_ref, "dx")
    check_grad(dWi, dWi_ref, "dW_init")


def test_backward_every_taped_variant():
    # Each forward variant that writes the tape, feeding the one backward kernel.
    srwm = _srwm()
    done = 0
    for v in srwm.variants():
        if not v["writes_tape"] or not srwm.backward_supported(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]):
            continue
        w = Workload("taped", B=2, H=2, d_in=v["d_in"], d_out=v["d_out"], T=45, io_dtype=v["io_dtype"],
                     apply_input_softmax=True, return_state=True, w0_std=v["d_in"] ** -0.5, seed=v["index"],
                     n_lr=v["n_lr"])
        say(f"[bwd] taped variant {v}")
        x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
        _, _, dx, dW0 = gpu_grads(w, x, W0, gy, gW, True, variant=v["index"])
        dx_ref, dW0_ref = oracle_bwd.grads(x, W0, True, gy, gW, n_lr=w.n_lr)
        check_grad(dx, dx_ref, f"variant {v['index']} dx")
        check_grad(dW0, dW0_ref, f"variant {v['index']} dW0")
        done += 1
    assert done >= 6


def test_backward_one_wave_taped_shorter_than_a_chunk():
    # One-wave taped units stage x a chunk of 16 or 32 steps at a time; a run
    # shorter than one chunk leaves the chunk's later rows unfetched and unused.
    srwm = _srwm()
    done = 0
    for v in srwm.variants():
        if v["waves"] != 1 or not v["writes_tape"] or not srwm.backward_supported(v["d_in"], v["d_out"],
                                                                                   v["io_dtype"], v["n_lr"]):
            continue
        for T in (1, 3):
            w = Workload("taped_short", B=2, H=2, d_in=v["d_in"], d_out=v["d_out"], T=T, io_dtype=v["io_dtype"],
                         apply_input_softmax=True, return_state=True, w0_std=v["d_in"] ** -0.5,
                         seed=100 + v["index"], n_lr=v["n_lr"])
            say(f"[bwd] one-wave taped variant {v['index']} T={T}")
            x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
            _, _, dx, dW0 = gpu_grads(w, x, W0, gy, gW, True, variant=v["index"])
            dx_ref, dW0_ref = oracle_bwd.grads(x, W0, True, gy, gW, n_lr=w.n_lr)
            check_grad(dx, dx_ref, f"variant {v['index']} T={T} dx")
            check_grad(dW0, dW0_ref, f"variant {v['index']} T={T} dW0")
            done += 1
    assert done >= 4


@pytest.mark.parametrize("n_lr", [4, 1])
@pytest.mark.parametrize("R", [0, 7])
def test_backward_kernel_by_unit_count(n_lr, R):
    # d = 64 has a 4-wave and an 8-wave backward kernel; B*H = 512 units take
    # the 4-wave one (the small shapes above take the 8-wave one).  Whole
    # sampled sequences against the oracle, with and without resets.
    srwm = _srwm()
    w = WORKLOADS["rl_d64_bf16"].with_(B=32, H=16, T=23, n_lr=n_lr)
    assert srwm.backward_resources(64, 64, n_lr, R > 0, w.units)["threads"] == 256
    assert srwm.backward_resources(64, 64, n_lr, R > 0, 4)["threads"] == 512
    flag = w.apply_input_softmax
    say(f"[bwd] 512 units n_lr={n_lr} R={R}")
    x, W0, gy = gen_x(w), gen_W0(w), gen_gy(w)
    _, _, dx, dWi = gpu_grads(w, x, W0, gy, None, flag, shared=False, reset_interval=R)
    for b in (0, 17, 31):
        dx_ref, dW_ref = oracle_bwd.grads(x[b:b + 1], W0, flag, gy[b:b + 1], None, n_lr=n_lr, reset_interval=R)
        check_grad(dx[b:b + 1], dx_ref, f"b={b} dx")
        check_grad(dWi[b], dW_ref, f"b={b} dW")


@pytest.mark.parametrize("name,bs", [("fewshot_d64", [0, 31]), ("rl_d64_bf16", [0, 127])])
def test_backward_full_size_sampled(name, bs):
    # The full workload on the GPU; whole sampled sequences (all heads, all T
    # steps) against the oracle.  Sequences are independent, so the per-unit
    # gradient of sequence b and dx[b] need only that sequence.
    w = WORKLOADS[name]
    flag = w.apply_input_softmax
    say(f"[bwd] full size {name}: B={w.B} H={w.H} T={w.T} (oracle on sequences {bs})")
    x, W0, gy = gen_x(w), gen_W0(w), gen_gy(w)
    _, _, dx, dWi = gpu_grads(w, x, W0, gy, None, flag, shared=False)
    assert np.isfinite(dx).all() and np.isfinite(dWi).all()
    for b in bs:
        dx_ref, dW_ref = oracle_bwd.grads(x[b:b + 1], W0, flag, gy[b:b + 1], None, n_lr=w.n_lr)
        rx = check_grad(dx[b:b + 1], dx_ref, f"{name} b={b} dx")
        rw = check_grad(dWi[b], dW_ref, f"{name} b={b} dW")
        say(f"[bwd] {name} b={b}: relL2 dx={rx:.2e} dW={rw:.2e}")


def test_backward_edge_cases():
    srwm = _srwm()
    w = WORKLOADS["multitask_d16"].with_(B=2, H=3)
    W0 = gen_W0(w)
    gW = gen_gW(w)
    # T = 0: W_T = W0, so dW_init = gW_T and dW0 = its sum over the batch.
    w0 = w.with_(T=0)
    _, _, dx, dWi = gpu_grads(w0, gen_x(w0), W0, gen_gy(w0), gW, False, shared=False)
    assert dx.shape == (2, 0, 3, 16)
    np.testing.assert_array_equal(dWi, gW)
    _, _, _, dW0 = gpu_grads(w0, gen_x(w0), W0, gen_gy(w0), gW, False, shared=True)
    np.testing.assert_allclose(dW0, gW.sum(0), rtol=1e-6, atol=0)
    # T = 1
    w1 = w.with_(T=1)
    x, gy = gen_x(w1), gen_gy(w1)
    _, _, dx, dW0 = gpu_grads(w1, x, W0, gy, gW, True)
    dx_ref, dW0_ref = oracle_bwd.grads(x, W0, True, gy, gW)
    check_grad(dx, dx_ref, "T=1 dx")
    check_grad(dW0, dW0_ref, "T=1 dW0")
    # B = 0: the shared gradient is zero
    wb = w.with_(B=0, T=5)
    xd = torch.zeros((0, 5, 3, 16), device=dev())
    y, WT, tape = srwm.forward(xd, to_dev(W0), save_tape=True)
    dx, dW0 = srwm.backward(xd, WT, tape, torch.zeros((0, 5, 3, 16), device=dev()), None)
    torch.cuda.synchronize()
    assert dx.shape == (0, 5, 3, 16) and dW0.shape == (3, wb.m, 16)
    assert (dW0 == 0).all()
    # zero cotangents give exactly zero gradients
    _, _, dx, dW0 = gpu_grads(w1, x, W0, np.zeros_like(gy), None, False)
    assert not dx.any() and not dW0.any()


def test_backward_deterministic():
    w = WORKLOADS["fewshot_d64"].with_(B=4, H=2, T=100)
    x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
    a = gpu_grads(w, x, W0, gy, gW, False)
    b = gpu_grads(w, x, W0, gy, gW, False)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("name", ["multitask_d16", "rl_d64_bf16"])
def test_autograd_function(name):
    # srwm.srwm(...) as a torch.autograd.Function: the same numbers as the
    # explicit forward/backward calls; gy or gW_T may be absent.
    srwm = _srwm()
    w = WORKLOADS[name].with_(B=2, H=2, T=60)
    flag = w.apply_input_softmax
    x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
    if w.io_dtype == "bf16":
        # y is bfloat16, so autograd hands the backward a bfloat16 cotangent
        gy = round_to_bf16(gy)
    _, _, dx_ref, dW_ref = gpu_grads(w, x, W0, gy, gW, flag)
    xd = to_dev(x, w.io_dtype).requires_grad_(True)
    Wd = to_dev(W0).requires_grad_(True)
    y, WT = srwm.srwm(xd, Wd, apply_input_softmax=flag)
    loss = (y.float() * to_dev(gy)).sum() + (WT * to_dev(gW)).sum()
    loss.backward()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(xd.grad.float().cpu().numpy(),
                                  torch.from_numpy(dx_ref).to(xd.dtype).float().numpy())
    np.testing.assert_array_equal(Wd.grad.cpu().numpy(), dW_ref)
    # only the final state in the loss
    xd.grad = None
    Wd.grad = None
    y, WT = srwm.srwm(xd, Wd, apply_input_softmax=flag)
    (WT * to_dev(gW)).sum().backward()
    torch.cuda.synchronize()
    dx_ref2, dW_ref2 = oracle_bwd.grads(x, W0, flag, np.zeros_like(gy), gW)
    check_grad(Wd.grad.cpu().numpy(), dW_ref2, "W_T-only dW0")
    if w.io_dtype == "f32":
        check_grad(xd.grad.cpu().numpy(), dx_ref2, "W_T-only dx")
    else:
        assert rel_l2(xd.grad.float().cpu().numpy(), dx_ref2) < 1e-2


# ---------------------------------------------------------------------------
# The reset ablation (review page Sec. 4.5): every R steps the state returns to
# the initial matrix.  The taped forward records each window's end state; the
# backward restarts every earlier window from it.
@pytest.mark.parametrize("name", [n for n in SMALL if n != "wide_d128"])  # no resets at d = 128
@pytest.mark.parametrize("n_lr", [4, 1])
@pytest.mark.parametrize("R", [1, 13])
def test_backward_reset_parity(name, n_lr, R):
    w = WORKLOADS[name].with_(n_lr=n_lr, **SMALL[name])
    flag = w.apply_input_softmax
    say(f"[bwd] reset R={R} {name} B={w.B} H={w.H} T={w.T} n_lr={n_lr}")
    x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
    y, WT, dx, dW0 = gpu_grads(w, x, W0, gy, gW, flag, reset_interval=R)
    y_ref, WT_ref = oracle.forward(x, W0, flag, n_lr=n_lr, reset_interval=R)
    check_y(y, y_ref, w.io_dtype, "taped forward with resets")
    check_state(WT, WT_ref, "taped forward with resets")
    dx_ref, dW0_ref = oracle_bwd.grads(x, W0, flag, gy, gW, n_lr=n_lr, reset_interval=R)
    rx = check_grad(dx, dx_ref, "dx")
    rw = check_grad(dW0, dW0_ref, "dW0")
    say(f"[bwd] relL2 dx={rx:.2e} dW0={rw:.2e}")


@pytest.mark.parametrize("name", ["fewshot_d64", "rl_d64_bf16"])
def test_window_states_are_window_end_states(name):
    # Window k covers steps [kR, (k+1)R) and starts from W0, so its end state
    # is the final state of a separate run over those steps alone.
    srwm = _srwm()
    w = WORKLOADS[name].with_(B=2, H=2, T=50)
    R = 13
    flag = w.apply_input_softmax
    x, W0 = gen_x(w), gen_W0(w)
    _, _, tape = srwm.forward(to_dev(x, w.io_dtype), to_dev(W0), apply_input_softmax=flag, reset_interval=R,
                              save_tape=True)
    torch.cuda.synchronize()
    ws = tape.window_states.cpu().numpy()
    assert ws.shape == (2, 2, (50 - 1) // R, w.m, w.d_in)
    for k in range(ws.shape[2]):
        _, ref = oracle.forward(np.ascontiguousarray(x[:, k * R:(k + 1) * R]), W0, flag)
        check_state(ws[:, :, k], ref, f"window {k} end state")


def test_backward_reset_longer_than_sequence():
    # R >= T: no reset happens and no window state is recorded; the gradient
    # is the plain one.
    w = WORKLOADS["fewshot_d64"].with_(B=2, H=2, T=30)
    x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
    _, _, dx, dW0 = gpu_grads(w, x, W0, gy, gW, False, reset_interval=30)
    _, _, dx1, dW01 = gpu_grads(w, x, W0, gy, gW, False)
    np.testing.assert_array_equal(dx, dx1)
    np.testing.assert_array_equal(dW0, dW01)


def test_backward_every_taped_reset_variant():
    srwm = _srwm()
    done = 0
    for v in srwm.variants():
        if not (v["writes_tape"] and v["supports_reset"]):
            continue
        w = Workload("taped_reset", B=2, H=2, d_in=v["d_in"], d_out=v["d_out"], T=45, io_dtype=v["io_dtype"],
                     apply_input_softmax=True, return_state=True, w0_std=v["d_in"] ** -0.5, seed=v["index"],
                     n_lr=v["n_lr"])
        say(f"[bwd] taped reset variant {v}")
        x, W0, gy, gW = gen_x(w), gen_W0(w), gen_gy(w), gen_gW(w)
        _, _, dx, dW0 = gpu_grads(w, x, W0, gy, gW, True, variant=v["index"], reset_interval=10)
        dx_ref, dW0_ref = oracle_bwd.grads(x, W0, True, gy, gW, n_lr=w.n_lr, reset_interval=10)
        check_grad(dx, dx_ref, f"variant {v['index']} dx")
        check_grad(dW0, dW0_ref, f"variant {v['index']} dW0")
        done += 1
    assert done >= 10


def test_autograd_with_resets():
    srwm = _srwm()
    w = WORKLOADS["fewshot_d64"].with_(B=2, H=2, T=40)
    x, W0, gy = gen_x(w), gen_W0(w), gen_gy(w)
    xd = to_dev(x).requires_grad_()
    W0d = to_dev(W0).requires_grad_()
    y, _ = srwm.srwm(xd, W0d, reset_interval=9)
    (y * to_dev(gy)).sum().backward()
    dx_ref, dW0_ref = oracle_bwd.grads(x, W0, False, gy, None, reset_interval=9)
    check_grad(xd.grad.cpu().numpy(), dx_ref, "autograd dx")
    check_grad(W0d.grad.cpu().numpy(), dW0_ref, "autograd dW0")


def test_backward_wide_full_size_sampled_unit():
    # The full wide workload (d = 128, T = 8192) through the wide backward
    # kernel; units are independent, so one sampled unit's gradients (its
    # sequence's dx for that head, its dW_init) are checked against the oracle
    # run on that unit alone.
    w = WORKLOADS["wide_d128"]
    flag = w.apply_input_softmax
    say(f"[bwd] full size wide_d128: B={w.B} H={w.H} T={w.T} (oracle on unit b=0, h=1)")
    x, W0, gy = gen_x(w), gen_W0(w), gen_gy(w)
    _, _, dx, dWi = gpu_grads(w, x, W0, gy, None, flag, shared=False)
    assert np.isfinite(dx).all() and np.isfinite(dWi).all()
    b, h = 0, 1
    dx_ref, dW_ref = oracle_bwd.grads(x[b:b + 1, :, h:h + 1], W0[h:h + 1], flag, gy[b:b + 1, :, h:h + 1], None,
                                      n_lr=w.n_lr)
    rx = check_grad(dx[b:b + 1, :, h:h + 1], dx_ref, "wide dx")
    rw = check_grad(dWi[b, h:h + 1], dW_ref, "wide dW")
    say(f"[bwd] wide_d128 unit ({b},{h}): relL2 dx={rx:.2e} dW={rw:.2e}")
