"""The Python binding on the GPU: buffers that do not start on a 16-byte
boundary are refused with a message naming the tensor, and library
temporaries stay valid while a caller's stream that is not torch's current
one still uses them."""
import numpy as np
import pytest
import torch

from self_referential_weight_amd.workloads import FWP_WORKLOADS, WORKLOADS, gen_gy, gen_W0, gen_x

pytestmark = pytest.mark.gpu


def _srwm():
    import self_referential_weight_amd as srwm
    return srwm


def say(msg):
    print(msg, flush=True)


def misaligned(t):
    """A contiguous copy of t that starts 4 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = flat[1:].view(t.shape)
    v.copy_(t)
    assert v.is_contiguous() and v.data_ptr() % 16 != 0
    return v


def test_misaligned_views_are_refused_by_name():
    srwm = _srwm()
    dev = torch.device("cuda:0")
    w = WORKLOADS["multitask_d16"].with_(B=2, T=5)
    say(f"[binding] misaligned views: {w}")
    x = torch.from_numpy(gen_x(w)).to(dev)
    W0 = torch.from_numpy(gen_W0(w)).to(dev)
    with pytest.raises(ValueError, match="x must start on a 16-byte boundary"):
        srwm.forward(misaligned(x), W0)
    with pytest.raises(ValueError, match="W0 must start on a 16-byte boundary"):
        srwm.forward(x, misaligned(W0))
    y, W_T, tape = srwm.forward(x, W0, save_tape=True)
    gy = torch.from_numpy(gen_gy(w)).to(dev)
    with pytest.raises(ValueError, match="gy must start on a 16-byte boundary"):
        srwm.backward(x, W_T, tape, misaligned(gy))
    f = FWP_WORKLOADS["deltanet_small"]
    z = torch.zeros((f.B, f.T, f.H, f.P), dtype=torch.float32, device=dev)
    yf = torch.empty((f.B, f.T, f.H, f.d_v), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="y must start on a 16-byte boundary"):
        srwm.fast_forward(z, f.d_key, f.d_v, y=misaligned(yf))
    # z's rows are read at any offset: a misaligned z is fine
    srwm.fast_forward(misaligned(z), f.d_key, f.d_v)
    # the aligned calls still run
    dx, dW0 = srwm.backward(x, W_T, tape, gy)
    srwm.fast_forward(z, f.d_key, f.d_v)
    torch.cuda.synchronize()
    assert torch.isfinite(dx).all() and torch.isfinite(dW0).all()


def _churn(shapes, dev):
    """Allocate and fill, on torch's current stream, tensors of the sizes the
    library's temporaries had: without a hold on their memory the caching
    allocator may hand those blocks out here while the kernels on the
    caller's stream still use them."""
    keep = []
    for _ in range(4):
        for s in shapes:
            keep.append(torch.full(s, float("nan"), dtype=torch.float32, device=dev))
    return keep


def test_srdeltanet_temporaries_on_a_non_current_stream():
    srwm = _srwm()
    dev = torch.device("cuda:0")
    w = FWP_WORKLOADS["srdeltanet_rl"].with_(B=32, T=512)
    say(f"[binding] srdeltanet carry buffers on a side stream: {w}")
    x = torch.from_numpy(gen_x(w)).to(dev)
    W0 = torch.from_numpy(gen_W0(w)).to(dev)
    y_ref, _, _, _ = srwm.srdeltanet_forward(x, W0, w.d_key, w.d_v, apply_input_softmax=w.apply_input_softmax,
                                             overlap=False)
    torch.cuda.synchronize()
    s, aux = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    assert s != torch.cuda.current_stream(dev)
    for _ in range(3):
        y, W_T, F_T, _ = srwm.srdeltanet_forward(x, W0, w.d_key, w.d_v, apply_input_softmax=w.apply_input_softmax,
                                                 stream=s, aux_stream=aux, chunk_steps=64)
        assert W_T is None and F_T is None
        keep = _churn([(w.B, w.H, w.m, w.d_in), (w.B, w.H, w.d_v, w.d_key)], dev)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        del keep


def test_backward_temporaries_on_a_non_current_stream():
    srwm = _srwm()
    dev = torch.device("cuda:0")
    w = WORKLOADS["fewshot_d64"].with_(T=96)
    say(f"[binding] backward per-unit gradients on a side stream: {w}")
    x = torch.from_numpy(gen_x(w)).to(dev)
    W0 = torch.from_numpy(gen_W0(w)).to(dev)
    gy = torch.from_numpy(gen_gy(w)).to(dev)
    y, W_T, tape = srwm.forward(x, W0, save_tape=True)
    dx_ref, dW0_ref = srwm.backward(x, W_T, tape, gy)
    torch.cuda.synchronize()
    s = torch.cuda.Stream(dev)
    for _ in range(3):
        dx, dW0 = srwm.backward(x, W_T, tape, gy, stream=s)
        keep = _churn([(w.B, w.H, w.m, w.d_in)], dev)
        torch.cuda.synchronize()
        assert torch.equal(dx, dx_ref) and torch.equal(dW0, dW0_ref)
        del keep
    assert np.isfinite(dW0.cpu().numpy()).all()
