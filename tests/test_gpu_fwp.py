"""GPU DeltaNet / SR-DeltaNet (through the C ABI) against the float64 oracle
on the same seeded inputs.  fp32 throughout; the tolerances of the SRWM
forward (tests/_parity.py) apply to y, the states and the projections z."""
import numpy as np
import pytest

from oracle import oracle
from self_referential_weight_amd.workloads import FWP_WORKLOADS, FwpWorkload, gen_W0, gen_W_slow, gen_x
from tests._parity import check_state, check_y, rel_l2

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _srwm():
    import self_referential_weight_amd as srwm
    return srwm


def dev():
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)


def td(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def run_deltanet(w, x, Wslow, F0=None):
    y, FT, z = _srwm().deltanet_forward(td(x), td(Wslow), w.d_key, w.d_v, F0=None if F0 is None else td(F0),
                                        return_state=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), FT.cpu().numpy(), z.cpu().numpy()


def run_srdeltanet(w, x, W0, F0=None):
    y, WT, FT, z = _srwm().srdeltanet_forward(td(x), td(W0), w.d_key, w.d_v, F0=None if F0 is None else td(F0),
                                              apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr,
                                              return_state=True)
    torch.cuda.synchronize()
    return y.cpu().numpy(), WT.cpu().numpy(), FT.cpu().numpy(), z.cpu().numpy()


def fast0(w, seed):
    return (np.random.default_rng([seed, 11]).standard_normal((w.B, w.H, w.d_v, w.d_key)) * 0.3).astype(np.float32)


# Shapes spanning several GEMM tiles with ragged edges (rows B*T, columns
# H*P, inner H*d_in not multiples of the tile sizes) and every fast kernel.
DN_CASES = [
    FwpWorkload("dn_d8", "deltanet", B=2, H=3, d_in=8, d_key=8, d_v=8, T=37, apply_input_softmax=False,
                w0_std=24 ** -0.5, seed=1),
    FwpWorkload("dn_d16", "deltanet", B=3, H=2, d_in=16, d_key=16, d_v=16, T=75, apply_input_softmax=False,
                w0_std=32 ** -0.5, seed=2),
    FwpWorkload("dn_d64", "deltanet", B=2, H=3, d_in=12, d_key=64, d_v=64, T=51, apply_input_softmax=False,
                w0_std=36 ** -0.5, seed=3),
]


@pytest.mark.parametrize("w", DN_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("with_f0", [False, True])
def test_deltanet_parity(w, with_f0):
    say(f"[fwp] deltanet {w}")
    x, Wslow = gen_x(w), gen_W_slow(w)
    F0 = fast0(w, w.seed) if with_f0 else None
    y, FT, z = run_deltanet(w, x, Wslow, F0)
    z_ref = (x.reshape(w.B * w.T, -1).astype(np.float64) @ Wslow.astype(np.float64).T).reshape(z.shape)
    assert rel_l2(z, z_ref) <= 1e-6
    y_ref, FT_ref = oracle.deltanet_forward(x, Wslow, w.d_key, w.d_v, F0=F0)
    check_y(y, y_ref, "f32", w.name)
    check_state(FT, FT_ref, w.name)


SDN_CASES = [
    FwpWorkload("sdn_d8", "srdeltanet", B=2, H=3, d_in=8, d_key=8, d_v=8, T=37, apply_input_softmax=False,
                w0_std=0.3, seed=4),
    FwpWorkload("sdn_d16", "srdeltanet", B=3, H=2, d_in=16, d_key=16, d_v=16, T=75, apply_input_softmax=True,
                w0_std=0.25, seed=5),
    FwpWorkload("sdn_d64", "srdeltanet", B=2, H=2, d_in=64, d_key=64, d_v=64, T=70, apply_input_softmax=True,
                w0_std=0.125, seed=6),
]


@pytest.mark.parametrize("w", SDN_CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("n_lr", [4, 1])
def test_srdeltanet_parity(w, n_lr):
    w = w.with_(n_lr=n_lr)
    say(f"[fwp] srdeltanet {w}")
    x, W0 = gen_x(w), gen_W0(w)
    F0 = fast0(w, w.seed)
    y, WT, FT, z = run_srdeltanet(w, x, W0, F0)
    z_ref, WT_ref = oracle.forward(x, W0, w.apply_input_softmax, n_lr=n_lr)
    check_y(z, z_ref, "f32", "SRWM projection")
    check_state(WT, WT_ref, "SRWM state")
    y_ref, WT2, FT_ref = oracle.srdeltanet_forward(x, W0, w.d_key, w.d_v, F0=F0,
                                                   apply_input_softmax=w.apply_input_softmax, n_lr=n_lr)
    check_y(y, y_ref, "f32", w.name)
    check_state(FT, FT_ref, w.name)


@pytest.mark.parametrize("name,bs", [("deltanet_rl", [0, 127]), ("srdeltanet_rl", [0, 127])])
def test_fwp_full_size_sampled(name, bs):
    w = FWP_WORKLOADS[name]
    say(f"[fwp] full size {name}: B={w.B} H={w.H} d={w.d_in} T={w.T} (oracle on sequences {bs})")
    x = gen_x(w)
    if w.kind == "deltanet":
        Wslow = gen_W_slow(w)
        y, FT, _ = run_deltanet(w, x, Wslow)
        for b in bs:
            y_ref, FT_ref = oracle.deltanet_forward(x[b:b + 1], Wslow, w.d_key, w.d_v)
            check_y(y[b:b + 1], y_ref, "f32", f"{name} b={b}")
            check_state(FT[b:b + 1], FT_ref, f"{name} b={b}")
            say(f"[fwp] {name} b={b}: relL2 y={rel_l2(y[b:b + 1], y_ref):.2e}")
    else:
        W0 = gen_W0(w)
        y, WT, FT, _ = run_srdeltanet(w, x, W0)
        for b in bs:
            y_ref, WT_ref, FT_ref = oracle.srdeltanet_forward(x[b:b + 1], W0, w.d_key, w.d_v,
                                                              apply_input_softmax=w.apply_input_softmax,
                                                              n_lr=w.n_lr)
            check_y(y[b:b + 1], y_ref, "f32", f"{name} b={b}")
            check_state(WT[b:b + 1], WT_ref, f"{name} b={b}")
            check_state(FT[b:b + 1], FT_ref, f"{name} b={b}")
            say(f"[fwp] {name} b={b}: relL2 y={rel_l2(y[b:b + 1], y_ref):.2e}")


def test_fwp_edge_cases():
    srwm = _srwm()
    w = DN_CASES[1]
    Wslow = gen_W_slow(w)
    F0 = fast0(w, 9)
    # T = 0: F_T = F0 (or zero), y empty
    x0 = np.zeros((w.B, 0, w.H, w.d_in), np.float32)
    y, FT, z = run_deltanet(w.with_(T=0), x0, Wslow, F0)
    assert y.shape == (w.B, 0, w.H, w.d_v)
    np.testing.assert_array_equal(FT, F0)
    y, FT, z = run_deltanet(w.with_(T=0), x0, Wslow)
    assert not FT.any()
    # B = 0
    y, FT, z = srwm.deltanet_forward(torch.zeros((0, 5, w.H, w.d_in), device=dev()), td(Wslow), w.d_key, w.d_v)
    torch.cuda.synchronize()
    assert y.shape == (0, 5, w.H, w.d_v)
    # continuation through the fast state: two calls equal one
    x = gen_x(w)
    y, FT, _ = run_deltanet(w, x, Wslow)
    ya, Fa, _ = run_deltanet(w.with_(T=30), np.ascontiguousarray(x[:, :30]), Wslow)
    yb, Fb, _ = run_deltanet(w.with_(T=w.T - 30), np.ascontiguousarray(x[:, 30:]), Wslow, Fa)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=1), y, rtol=0, atol=1e-6 * np.abs(y).max())
    np.testing.assert_allclose(Fb, FT, rtol=0, atol=1e-6 * np.abs(FT).max())
    # SR-DeltaNet with T = 0: both states pass through
    ws = SDN_CASES[1]
    W0 = gen_W0(ws)
    y, WT, FT, z = run_srdeltanet(ws.with_(T=0), np.zeros((ws.B, 0, ws.H, ws.d_in), np.float32), W0, F0)
    np.testing.assert_array_equal(WT, np.broadcast_to(W0, WT.shape))
    np.testing.assert_array_equal(FT, F0)


def test_fwp_deterministic():
    w = DN_CASES[2]
    x, Wslow = gen_x(w), gen_W_slow(w)
    a = run_deltanet(w, x, Wslow)
    b = run_deltanet(w, x, Wslow)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_split_entry_points_equal_the_composites():
    # projection + fast recurrence called separately give the composite's bits
    srwm = _srwm()
    w = DN_CASES[2]
    x, Wslow = gen_x(w), gen_W_slow(w)
    F0 = fast0(w, 13)
    y, FT, z = run_deltanet(w, x, Wslow, F0)
    z2 = srwm.deltanet_project(td(x), td(Wslow), w.d_key, w.d_v)
    y2, F2 = srwm.fast_forward(z2, w.d_key, w.d_v, F0=td(F0), return_state=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(z2.cpu().numpy(), z)
    np.testing.assert_array_equal(y2.cpu().numpy(), y)
    np.testing.assert_array_equal(F2.cpu().numpy(), FT)
    ws = SDN_CASES[2]
    x, W0 = gen_x(ws), gen_W0(ws)
    y, WT, FT, z = run_srdeltanet(ws, x, W0)
    zs, _ = srwm.forward(td(x), td(W0), apply_input_softmax=ws.apply_input_softmax, n_lr=ws.n_lr)
    y3, F3 = srwm.fast_forward(zs, ws.d_key, ws.d_v, return_state=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(zs.cpu().numpy(), z)
    np.testing.assert_array_equal(y3.cpu().numpy(), y)
    np.testing.assert_array_equal(F3.cpu().numpy(), FT)


def _srdeltanet_t(w, x, W0, F0, **kw):
    return _srwm().srdeltanet_forward(x, W0, w.d_key, w.d_v, F0=F0, apply_input_softmax=w.apply_input_softmax,
                                      n_lr=w.n_lr, return_state=True, **kw)


@pytest.mark.parametrize("w", SDN_CASES[1:], ids=lambda w: w.name)
@pytest.mark.parametrize("chunk", [1, 7, 32, 69])
def test_srdeltanet_overlap_same_bits(w, chunk):
    # The projection of later steps on the caller's stream beside the fast
    # matrix of earlier ones on a second stream, states carried in W_T and F_T
    # between chunks: the one-stream call's bits, ragged last chunks included.
    say(f"[fwp] srdeltanet overlapped, chunks of {chunk}: {w}")
    x, W0 = td(gen_x(w)), td(gen_W0(w))
    for F0 in (None, td(fast0(w, 21))):
        ref = _srdeltanet_t(w, x, W0, F0, overlap=False)
        got = _srdeltanet_t(w, x, W0, F0, chunk_steps=chunk)
        torch.cuda.synchronize()
        for name, a, b in zip(("y", "W_T", "F_T", "z"), ref, got):
            assert torch.equal(a, b), f"{name} differs, chunks of {chunk}"


def test_srdeltanet_overlap_full_size_and_stream_order():
    # The RL-sized workload chunked automatically, on a caller stream that is
    # not torch's current one: work queued on that stream right after the call
    # (a copy of y and F_T) sees the fast matrix's last chunk, which ran on the
    # second stream.
    w = FWP_WORKLOADS["srdeltanet_rl"]
    say(f"[fwp] srdeltanet full size overlapped: {w}")
    x, W0 = td(gen_x(w)), td(gen_W0(w))
    ref = _srdeltanet_t(w, x, W0, None, overlap=False)
    torch.cuda.synchronize()
    s, aux = torch.cuda.Stream(dev()), torch.cuda.Stream(dev())
    s.wait_stream(torch.cuda.current_stream(dev()))
    with torch.cuda.stream(s):
        got = _srdeltanet_t(w, x, W0, None, stream=s, aux_stream=aux)
        y_copy, F_copy = got[0].clone(), got[2].clone()
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "W_T", "F_T", "z"), ref, got):
        assert torch.equal(a, b), f"{name} differs"
    assert torch.equal(y_copy, ref[0]) and torch.equal(F_copy, ref[2])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("d", [16, 64])
def test_forward_over_time_slices(io, d):
    # Steps [0, t1) and then [t1, T) of one x and one y buffer (views along
    # time, no copies), the second call starting from the first's W_T, give
    # the bits of one call over all T steps.
    srwm = _srwm()
    from self_referential_weight_amd.workloads import Workload, gen_W0 as gen_W0_srwm, gen_x as gen_x_srwm
    w = Workload(f"slices_d{d}", B=3, H=2, d_in=d, d_out=d, T=75, io_dtype=io, apply_input_softmax=d == 64,
                 return_state=True, w0_std=d ** -0.5)
    say(f"[fwp] forward over time slices: {w}")
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    x = torch.from_numpy(gen_x_srwm(w)).to(dev()).to(dt)
    W0 = td(gen_W0_srwm(w))
    y_ref, W_ref = srwm.forward(x, W0, apply_input_softmax=w.apply_input_softmax, return_state=True)
    y = torch.full_like(y_ref, float("nan"))
    for t1 in (1, 30, 74):
        _, Wa = srwm.forward(x[:, :t1], W0, apply_input_softmax=w.apply_input_softmax, y=y[:, :t1],
                             return_state=True)
        _, Wb = srwm.forward(x[:, t1:], Wa, apply_input_softmax=w.apply_input_softmax, y=y[:, t1:],
                             return_state=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(Wb, W_ref), f"split at {t1}"
    with pytest.raises(ValueError):
        srwm.forward(x[:, 5:9], W0)  # a time slice needs its y slice


def test_fast_forward_over_time_slices():
    srwm = _srwm()
    w = SDN_CASES[2]
    z = torch.randn((w.B, w.T, w.H, w.P), generator=torch.Generator().manual_seed(5)).to(dev()) * 0.5
    y_ref, F_ref = srwm.fast_forward(z, w.d_key, w.d_v, return_state=True)
    y = torch.full_like(y_ref, float("nan"))
    _, Fa = srwm.fast_forward(z[:, :33], w.d_key, w.d_v, y=y[:, :33], return_state=True)
    _, Fb = srwm.fast_forward(z[:, 33:], w.d_key, w.d_v, F0=Fa, y=y[:, 33:], return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(Fb, F_ref)


@pytest.mark.parametrize("B", [260])
def test_fast_kernel_for_many_units(B):
    # Above 512 units the fast matrix runs on 4 row-holding waves per unit (one
    # row of 16 columns per lane) beside 4 preparing ones instead of 8 beside 4: the same
    # results, checked against the oracle on sampled sequences, with a ragged
    # last chunk (T = 37).
    w = FwpWorkload("dn_units", "deltanet", B=B, H=2, d_in=16, d_key=64, d_v=64, T=37, apply_input_softmax=False,
                    w0_std=32 ** -0.5, seed=7)
    say(f"[fwp] fast kernel, {w.B * w.H} units: {w}")
    x, Wslow = gen_x(w), gen_W_slow(w)
    F0 = fast0(w, 17)
    y, FT, _ = run_deltanet(w, x, Wslow, F0)
    for b in (0, 131, B - 1):
        y_ref, FT_ref = oracle.deltanet_forward(x[b:b + 1], Wslow, w.d_key, w.d_v, F0=F0[b:b + 1])
        check_y(y[b:b + 1], y_ref, "f32", f"{w.name} b={b}")
        check_state(FT[b:b + 1], FT_ref, f"{w.name} b={b}")
