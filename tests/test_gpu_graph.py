"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): no
kernel here records a memset or allocates, so a captured forward, backward
or DeltaNet call replays to the eager result.  Each replay is checked, with
eager work and synchronisations in between."""
import numpy as np
import pytest

from self_referential_weight_amd.workloads import FWP_WORKLOADS, WORKLOADS, gen_gy, gen_W0, gen_W_slow, gen_x

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _srwm():
    import self_referential_weight_amd as srwm
    return srwm


def td(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
    return t.to(dtype) if dtype is not None else t


def replay_and_check(capture, outputs_eager, n=3):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture()  # warm-up outside the graph on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = capture()
    for i in range(n):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, outputs_eager):
            assert torch.equal(o, e), f"replay {i} differs from the eager result"
        # eager work between replays
        (torch.randn(1024, device="cuda:0") * 2).sum().item()


def test_forward_in_graph():
    srwm = _srwm()
    w = WORKLOADS["fewshot_d64"].with_(B=4, T=100)
    x, W0 = td(gen_x(w)), td(gen_W0(w))
    y_e, WT_e = srwm.forward(x, W0, return_state=True)
    y = torch.empty_like(y_e)
    WT = torch.empty_like(WT_e)

    def capture():
        srwm.forward(x, W0, return_state=True, y=y, W_T=WT)
        return (y, WT)
    replay_and_check(capture, (y_e, WT_e))


def test_training_step_in_graph():
    srwm = _srwm()
    w = WORKLOADS["multitask_d16"].with_(B=2, T=64)
    x, W0, gy = td(gen_x(w)), td(gen_W0(w)), td(gen_gy(w))
    y_e, WT_e, tape = srwm.forward(x, W0, save_tape=True)
    dx_e, dW_e = srwm.backward(x, WT_e, tape, gy)
    torch.cuda.synchronize()

    def capture():
        y, WT, tp = srwm.forward(x, W0, save_tape=True)
        dx, dW = srwm.backward(x, WT, tp, gy)
        return (y, WT, dx, dW)
    replay_and_check(capture, (y_e, WT_e, dx_e, dW_e))


def test_deltanet_in_graph():
    srwm = _srwm()
    f = FWP_WORKLOADS["deltanet_small"]
    x, Ws = td(gen_x(f)), td(gen_W_slow(f))
    y_e, FT_e, z_e = srwm.deltanet_forward(x, Ws, f.d_key, f.d_v, return_state=True)
    torch.cuda.synchronize()

    def capture():
        return srwm.deltanet_forward(x, Ws, f.d_key, f.d_v, return_state=True)
    replay_and_check(capture, (y_e, FT_e, z_e))


def test_srdeltanet_overlapped_in_graph():
    # The two-stream chunk schedule captured from the caller's stream: the
    # second stream joins the capture through the schedule's events and is
    # joined back at its end, so the graph replays to the one-stream result.
    srwm = _srwm()
    w = FWP_WORKLOADS["srdeltanet_small"].with_(d_in=64, d_key=64, d_v=64, T=100, B=2)
    x, W0 = td(gen_x(w)), td(gen_W0(w))
    kw = dict(apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr, return_state=True)
    y_e, WT_e, FT_e, z_e = srwm.srdeltanet_forward(x, W0, w.d_key, w.d_v, overlap=False, **kw)
    torch.cuda.synchronize()
    aux = torch.cuda.Stream()
    z, y = torch.empty_like(z_e), torch.empty_like(y_e)

    def capture():
        y_, WT, FT, z_ = srwm.srdeltanet_forward(x, W0, w.d_key, w.d_v, z=z, y=y, aux_stream=aux, chunk_steps=23,
                                                 **kw)
        return (y_, WT, FT, z_)
    replay_and_check(capture, (y_e, WT_e, FT_e, z_e))
