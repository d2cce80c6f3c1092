"""MI355X-native forward recurrence of the multi-head, 4-learning-rate
self-referential weight matrix (SRWM).

``forward`` is a thin binding over ``srwm_forward`` of libsrwm (include/srwm.h):
it checks and marshals torch device tensors and the current HIP stream; every
step of the recurrence runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: without the built library, or with tensors off the GPU, the
call raises.
"""
from __future__ import annotations

from typing import NamedTuple, Optional

from . import _lib
from .workloads import HEADLINE, WORKLOADS, Workload

__all__ = ["forward", "backward", "srwm", "Tape", "tape_row", "deltanet_forward", "deltanet_project", "fast_forward", "srdeltanet_forward", "srdeltanet_chunk_steps", "fwp_supported", "supported", "backward_supported", "variants", "select_variant", "kernel_resources", "backward_resources", "m_rows", "WORKLOADS", "HEADLINE", "Workload"]


def m_rows(d_in: int, d_out: int, n_lr: int = 4) -> int:
    """Rows of the state: d_out + 2*d_in + n_lr (y, k, q blocks and the rate logits)."""
    return d_out + 2 * d_in + n_lr


def _io(io_dtype: str) -> int:
    return _lib.SRWM_IO_BF16 if io_dtype == "bf16" else _lib.SRWM_IO_F32


def supported(d_in: int, d_out: int, io_dtype: str = "f32", n_lr: int = 4) -> bool:
    return bool(_lib.load().srwm_supported(d_in, d_out, _io(io_dtype), n_lr))


def backward_supported(d_in: int, d_out: int, io_dtype: str = "f32", n_lr: int = 4) -> bool:
    return bool(_lib.load().srwm_backward_supported(d_in, d_out, _io(io_dtype), n_lr))


def variants() -> list[dict]:
    return _lib.variants()


def kernel_resources(variant: int) -> dict:
    """Registers, LDS, scratch and occupancy of forward variant `variant` on the
    current device (vgprs, lds_bytes, scratch_bytes, threads, workgroups_per_cu,
    waves_per_simd)."""
    return _lib.variant_resources(variant)


def backward_resources(d_in: int, d_out: int, n_lr: int = 4, reset: bool = False, units: int = 2048) -> dict:
    """The same for the kernel srwm_backward launches for this shape and B*H = units."""
    return _lib.backward_resources(d_in, d_out, n_lr, reset, units)


def select_variant(d_in: int, d_out: int, io_dtype: str, units: int, n_lr: int = 4,
                   reset_interval: int = 0) -> dict:
    """The kernel variant the automatic choice uses for B*H = units."""
    i = _lib.load().srwm_select_variant(d_in, d_out, _io(io_dtype), n_lr, reset_interval, units)
    if i < 0:
        raise RuntimeError(_lib.strerror(i))
    return _lib.variants()[i]


class Tape(NamedTuple):
    """What ``forward(..., save_tape=True)`` records for ``backward``.

    rows: [B, H, T, tape_row] float32, one row per unit and step (a_t,
    phi(k_t), phi(q_t) - phi(k_t), the learning rates, u_t).
    window_states: with reset_interval R > 0, the end state of every window
    but the last, [B, H, (T - 1) // R, m, d_in] float32; else None.
    """
    rows: object
    window_states: Optional[object]
    reset_interval: int


def tape_row(d_in: int, d_out: int, n_lr: int = 4) -> int:
    """Floats per step and unit in the backward tape."""
    return int(_lib.load().srwm_tape_row(d_in, d_out, n_lr))


def forward(x, W0, apply_input_softmax: bool = False, return_state: bool = False,
            variant: int = -1, y=None, W_T=None, stream=None, n_lr: int = 4,
            reset_interval: int = 0, save_tape: bool = False):
    """Run the SRWM recurrence on the GPU.

    x   : torch tensor [B, T, H, d_in], float32 or bfloat16, on a ROCm device
    W0  : torch float32 tensor [H, m, d_in] (shared over the batch) or
          [B, H, m, d_in] (one initial state per sequence, e.g. an earlier
          W_T), m = d_out + 2*d_in + n_lr, same device
    n_lr: 4 (a learning rate per row block) or 1 (one for every row)
    reset_interval: 0, or R > 0 to return every state to W0 before each step
          t > 0 with t % R == 0 (the reset ablation)
    save_tape: also record what ``backward`` needs (implies return_state);
          the return value is then (y, W_T, Tape).
    Returns (y [B, T, H, d_out] in x's dtype, W_T [B, H, m, d_in] float32 or None).
    ``y`` / ``W_T`` may be passed preallocated; the call is asynchronous on
    ``stream`` (default: torch's current stream).
    """
    import torch

    lib = _lib.load()
    if not (isinstance(x, torch.Tensor) and isinstance(W0, torch.Tensor)):
        raise TypeError("x and W0 must be torch tensors")
    if x.device.type != "cuda" or W0.device != x.device:
        raise ValueError("x and W0 must live on the same ROCm GPU")
    if x.dtype == torch.float32:
        io = _lib.SRWM_IO_F32
    elif x.dtype == torch.bfloat16:
        io = _lib.SRWM_IO_BF16
    else:
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    if W0.dtype != torch.float32:
        raise TypeError("W0 must be float32")
    if x.dim() != 4 or W0.dim() not in (3, 4):
        raise ValueError("x must be [B,T,H,d_in] and W0 [H,m,d_in] or [B,H,m,d_in]")
    t_stride = _time_stride(x, "x")
    if not W0.is_contiguous():
        raise ValueError("W0 must be contiguous")
    B, T, H, d_in = x.shape
    per_seq = W0.dim() == 4
    if per_seq:
        B2, H2, m, d_in2 = W0.shape
        if B2 != B:
            raise ValueError(f"per-sequence W0 has batch {B2}, x has {B}")
    else:
        H2, m, d_in2 = W0.shape
    if H2 != H or d_in2 != d_in:
        raise ValueError(f"W0 shape {tuple(W0.shape)} does not match x {tuple(x.shape)}")
    d_out = m - 2 * d_in - n_lr
    if d_out < 1:
        raise ValueError(f"W0 has {m} rows; need d_out + 2*d_in + {n_lr} with d_out >= 1")
    if y is None:
        if t_stride:
            raise ValueError("x is a time slice of longer sequences: pass y, a slice of the same steps")
        y = torch.empty((B, T, H, d_out), dtype=x.dtype, device=x.device)
    elif (tuple(y.shape) != (B, T, H, d_out) or y.dtype != x.dtype or y.device != x.device
          or _time_stride(y, "y") != t_stride):
        raise ValueError("preallocated y has the wrong shape/dtype/device/layout")
    if save_tape:
        return_state = True
    if return_state:
        if W_T is None:
            W_T = torch.empty((B, H, m, d_in), dtype=torch.float32, device=x.device)
        elif (tuple(W_T.shape) != (B, H, m, d_in) or W_T.dtype != torch.float32
              or W_T.device != x.device or not W_T.is_contiguous()):
            raise ValueError("preallocated W_T has the wrong shape/dtype/device/layout")
    else:
        W_T = None
    tape = wstates = None
    if save_tape:
        tape = torch.empty((B, H, T, tape_row(d_in, d_out, n_lr)), dtype=torch.float32, device=x.device)
        if reset_interval > 0:
            n_res = (T - 1) // reset_interval if T > 0 else 0
            wstates = torch.empty((B, H, n_res, m, d_in), dtype=torch.float32, device=x.device)
    _check_aligned(x=x, W0=W0, y=y, W_T=W_T)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    a = _lib.ForwardArgs(
        x=x.data_ptr() if x.numel() else None, W0=W0.data_ptr() if W0.numel() else None,
        y=y.data_ptr() if y.numel() else None,
        W_T=W_T.data_ptr() if W_T is not None and W_T.numel() else None,
        B=B, T=T, H=H, d_in=d_in, d_out=d_out, m=m, io_dtype=io,
        apply_input_softmax=int(bool(apply_input_softmax)), n_lr=int(n_lr),
        w0_per_sequence=int(per_seq), reset_interval=int(reset_interval), variant=int(variant),
        stream=handle, tape=tape.data_ptr() if tape is not None and tape.numel() else None,
        window_states=wstates.data_ptr() if wstates is not None and wstates.numel() else None,
        t_stride=t_stride)
    with torch.cuda.device(x.device):
        rc = lib.srwm_forward_ex(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    if save_tape:
        return y, W_T, Tape(tape, wstates, int(reset_interval))
    return y, W_T


def backward(x, W_T, tape, gy, gW_T=None, apply_input_softmax: bool = False, n_lr: int = 4,
             shared_W0: bool = True, stream=None, no_alloc: bool = False):
    """Gradients of L = sum_t <gy[t], y_t> + <gW_T, W_T> through the recurrence.

    x, W_T, tape: the forward pass's input, final state and Tape
    (``forward(..., save_tape=True)``, with or without a reset interval); gy
    [B, T, H, d_out] and gW_T [B, H, m, d_in] (or None) float32.  Returns
    (dx [B, T, H, d_in] float32, dW0): dW0 is [H, m, d_in] (summed over the
    batch) when shared_W0, else the per-unit gradient [B, H, m, d_in].
    no_alloc (with shared_W0): call srwm_backward_noalloc, whose per-unit
    gradients live in the library's scratch array instead of a temporary
    (calls that overlap in time on one GPU must not both use it).
    """
    import torch

    lib = _lib.load()
    if not isinstance(tape, Tape):
        raise TypeError("tape must be the Tape that forward(..., save_tape=True) returned")
    wstates, reset_interval = tape.window_states, tape.reset_interval
    tape = tape.rows
    B, T, H, d_in = x.shape
    m = W_T.shape[-2]
    d_out = m - 2 * d_in - n_lr
    if x.device.type != "cuda":
        raise ValueError("x must live on a ROCm GPU")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"x must be float32 or bfloat16, got {x.dtype}")
    io = _lib.SRWM_IO_BF16 if x.dtype == torch.bfloat16 else _lib.SRWM_IO_F32
    if gW_T is not None and (gW_T.dtype != torch.float32 or tuple(gW_T.shape) != (B, H, m, d_in)):
        raise ValueError("gW_T must be float32 [B, H, m, d_in]")
    for name, t_ in (("x", x), ("W_T", W_T), ("tape", tape), ("gy", gy)) + ((("gW_T", gW_T),) if gW_T is not None else ()):
        if t_.device != x.device or not t_.is_contiguous():
            raise ValueError(f"{name} must be contiguous on x's device")
    if gy.dtype != torch.float32 or W_T.dtype != torch.float32 or tape.dtype != torch.float32:
        raise TypeError("gy, W_T and tape must be float32")
    if tuple(gy.shape) != (B, T, H, d_out) or tuple(W_T.shape) != (B, H, m, d_in):
        raise ValueError("gy / W_T shapes do not match x")
    if tuple(tape.shape) != (B, H, T, tape_row(d_in, d_out, n_lr)):
        raise ValueError("tape shape does not match x")
    if reset_interval > 0:
        n_res = (T - 1) // reset_interval if T > 0 else 0
        if (wstates is None or tuple(wstates.shape) != (B, H, n_res, m, d_in) or wstates.dtype != torch.float32
                or wstates.device != x.device or not wstates.is_contiguous()):
            raise ValueError("the tape's window states do not match x")
    _check_aligned(W_T=W_T, tape=tape, gy=gy, gW_T=gW_T, window_states=wstates)
    if no_alloc and not shared_W0:
        raise ValueError("no_alloc returns only the batch-summed gradient: it needs shared_W0=True")
    dx = torch.empty((B, T, H, d_in), dtype=torch.float32, device=x.device)
    dWi = None if no_alloc else torch.empty((B, H, m, d_in), dtype=torch.float32, device=x.device)
    dW0 = torch.empty((H, m, d_in), dtype=torch.float32, device=x.device) if shared_W0 else None
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def ptr(t_):
        return t_.data_ptr() if t_ is not None and t_.numel() else None

    # x gives the shapes, dtype and device; the kernels read u_t from the tape
    a = _lib.BackwardArgs(x=None, W_T=ptr(W_T), tape=ptr(tape), gy=ptr(gy), gW_T=ptr(gW_T),
                          dx=ptr(dx), dW_init=ptr(dWi), dW0=ptr(dW0), B=B, T=T, H=H, d_in=d_in,
                          d_out=d_out, m=m, io_dtype=io,
                          apply_input_softmax=int(bool(apply_input_softmax)), n_lr=int(n_lr),
                          stream=handle, reset_interval=int(reset_interval), window_states=ptr(wstates))
    with torch.cuda.device(x.device):
        rc = lib.srwm_backward_noalloc(a) if no_alloc else lib.srwm_backward(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    if shared_W0:
        _hold_for(dWi, x.device, stream)  # per-unit gradients, summed into dW0 on `stream`
    return dx, (dW0 if shared_W0 else dWi)


def _autograd_function():
    import torch

    class SRWMFunction(torch.autograd.Function):
        """y, W_T = srwm(x, W0) with gradients for x and W0 from ``backward``."""

        @staticmethod
        def forward(ctx, x, W0, apply_input_softmax, n_lr, reset_interval):
            y, W_T, tape = forward(x, W0, apply_input_softmax=apply_input_softmax, n_lr=n_lr,
                                   reset_interval=reset_interval, save_tape=True)
            ws = tape.window_states if tape.window_states is not None else W_T.new_empty(0)
            ctx.save_for_backward(x, W_T, tape.rows, ws)
            ctx.flags = (bool(apply_input_softmax), int(n_lr), W0.dim() == 3, int(reset_interval))
            ctx.set_materialize_grads(False)
            return y, W_T

        @staticmethod
        def backward(ctx, gy, gW_T):
            x, W_T, rows, ws = ctx.saved_tensors
            flag, n_lr, shared, reset_interval = ctx.flags
            tape = Tape(rows, ws if reset_interval > 0 else None, reset_interval)
            if gy is None:
                d_out = W_T.shape[-2] - 2 * x.shape[-1] - n_lr
                gy = torch.zeros((*x.shape[:3], d_out), dtype=torch.float32, device=x.device)
            else:
                gy = gy.float().contiguous()
            gW_T = None if gW_T is None else gW_T.contiguous()
            dx, dW0 = backward(x, W_T, tape, gy, gW_T, apply_input_softmax=flag, n_lr=n_lr,
                               shared_W0=shared)
            return dx.to(x.dtype), dW0, None, None, None

    return SRWMFunction


def srwm(x, W0, apply_input_softmax: bool = False, n_lr: int = 4, reset_interval: int = 0):
    """Differentiable forward: returns (y, W_T); gradients flow to x and W0."""
    return _autograd_function().apply(x, W0, apply_input_softmax, n_lr, reset_interval)


def fwp_supported(d_key: int, d_v: int) -> bool:
    """Whether the fast-matrix kernel of DeltaNet / SR-DeltaNet exists for (d_key, d_v)."""
    return bool(_lib.load().srwm_fwp_supported(d_key, d_v))


def _fwp_common(x, F0, d_key, d_v, return_state, z, y):
    import torch

    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a torch tensor on a ROCm GPU")
    if x.dtype != torch.float32 or x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous float32 [B, T, H, d_in] tensor")
    B, T, H, d_in = x.shape
    P = d_v + 2 * d_key + 1
    if F0 is not None and (tuple(F0.shape) != (B, H, d_v, d_key) or F0.dtype != torch.float32
                           or F0.device != x.device or not F0.is_contiguous()):
        raise ValueError("F0 must be a contiguous float32 [B, H, d_v, d_key] tensor on x's device")
    if z is None:
        z = torch.empty((B, T, H, P), dtype=torch.float32, device=x.device)
    elif tuple(z.shape) != (B, T, H, P) or z.dtype != torch.float32 or not z.is_contiguous():
        raise ValueError("z must be a contiguous float32 [B, T, H, P] tensor")
    if y is None:
        y = torch.empty((B, T, H, d_v), dtype=torch.float32, device=x.device)
    elif tuple(y.shape) != (B, T, H, d_v) or y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError("y must be a contiguous float32 [B, T, H, d_v] tensor")
    F_T = torch.empty((B, H, d_v, d_key), dtype=torch.float32, device=x.device) if return_state else None
    return B, T, H, d_in, P, z, y, F_T


def _time_stride(t, name: str) -> int:
    """0 for a contiguous [B, T, H, D] tensor; S for the steps [t0, t0+T) of a
    contiguous [B, S, H, D] buffer (a slice along dim 1); ValueError else."""
    if t.is_contiguous():
        return 0
    B, T, H, D = t.shape
    st = t.stride()
    if st[3] == 1 and st[2] == D and st[1] == H * D and st[0] % max(H * D, 1) == 0 and st[0] // (H * D) >= T:
        return st[0] // (H * D)
    raise ValueError(f"{name} must be contiguous or a time slice [:, t0:t1] of a contiguous [B, S, H, D] tensor")


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() else None


def _check_aligned(**tensors):
    """The kernels move 16-byte pieces, so the library takes only buffers that
    start on a 16-byte boundary (a misaligned pointer is SRWM_ERR_ARG); name
    the offending tensor here instead."""
    for name, t in tensors.items():
        if t is not None and t.numel() and t.data_ptr() % 16:
            raise ValueError(f"{name} must start on a 16-byte boundary (libsrwm's kernels move 16-byte pieces); "
                             f"its data pointer is {t.data_ptr() % 16} bytes past one, as a view at an odd "
                             f"offset into a larger buffer can be: pass a fresh allocation or .clone() it")


def _stream_handle(x, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _hold_for(t, device, *streams):
    """Keep the caching allocator from handing `t`'s memory to other work
    until what is queued now on each of `streams` (torch streams or raw HIP
    handles) has run: for library temporaries that are dropped when the call
    returns while kernels that use them may still be queued on a stream other
    than torch's current one."""
    import torch

    if t is None or not t.numel():
        return
    for s in streams:
        if s is None:
            continue
        if not hasattr(s, "cuda_stream"):
            s = torch.cuda.ExternalStream(int(s), device=device)
        t.record_stream(s)


def deltanet_forward(x, W_slow, d_key: int, d_v: int, F0=None, return_state: bool = False, z=None, y=None,
                     stream=None):
    """DeltaNet forward on the GPU (full-width slow projection, fast matrix
    queried after its delta write).

    x [B, T, H, d_in] float32; W_slow [H*P, H*d_in] float32 with
    P = d_v + 2*d_key + 1 (head h's rows [h*P, (h+1)*P) give [k; v; q; beta]);
    F0 [B, H, d_v, d_key] or None (zero).  Returns (y [B, T, H, d_v],
    F_T [B, H, d_v, d_key] or None, z [B, T, H, P] the projections).
    """
    import torch

    lib = _lib.load()
    B, T, H, d_in, P, z, y, F_T = _fwp_common(x, F0, d_key, d_v, return_state, z, y)
    if (tuple(W_slow.shape) != (H * P, H * d_in) or W_slow.dtype != torch.float32
            or W_slow.device != x.device or not W_slow.is_contiguous()):
        raise ValueError("W_slow must be a contiguous float32 [H*P, H*d_in] tensor on x's device")
    _check_aligned(x=x, W_slow=W_slow, F0=F0, z=z, y=y)
    a = _lib.DeltanetArgs(x=_ptr(x), W_slow=_ptr(W_slow), F0=_ptr(F0), z=_ptr(z), y=_ptr(y), F_T=_ptr(F_T),
                          B=B, T=T, H=H, d_in=d_in, d_key=d_key, d_v=d_v, stream=_stream_handle(x, stream))
    with torch.cuda.device(x.device):
        rc = lib.srwm_deltanet_forward(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    return y, F_T, z


_aux_streams: dict = {}


def _aux_stream(device):
    """The binding's second stream on `device` (default priority), made once."""
    import torch

    key = torch.device(device).index
    if key not in _aux_streams:
        _aux_streams[key] = torch.cuda.Stream(device)
    return _aux_streams[key]


def srdeltanet_forward(x, W0, d_key: int, d_v: int, F0=None, apply_input_softmax: bool = False,
                       n_lr: int = 4, return_state: bool = False, z=None, y=None, stream=None,
                       overlap: bool = True, aux_stream=None, chunk_steps: int = 0):
    """SR-DeltaNet forward on the GPU: a per-head SRWM (d_out = P) produces
    each step's [k; v; q; beta] for a fast matrix queried after its write.

    W0 [H, m, d_in] float32, m = P + 2*d_in + n_lr.  Returns (y, W_T (the
    SRWM's final state [B, H, m, d_in]) or None, F_T or None, z).
    overlap: run the projection of later steps beside the fast matrix of
    earlier ones on a second stream (``aux_stream``, default the binding's
    own), in chunks of ``chunk_steps`` (0: the library's choice; T or more:
    no overlap).  Same results either way; the states of both halves are
    then carried in W_T and F_T, allocated here when not returned.
    """
    import torch

    lib = _lib.load()
    if overlap:
        B_, T_, H_, d_in_ = x.shape
        C = chunk_steps or lib.srwm_srdeltanet_chunk_steps(B_, T_, H_, d_in_, d_key, d_v, n_lr)
        overlap = 0 < C < T_  # else one stream (errors are reported by the call below)
    B, T, H, d_in, P, z, y, F_T = _fwp_common(x, F0, d_key, d_v, return_state or overlap, z, y)
    m = P + 2 * d_in + n_lr
    if (tuple(W0.shape) != (H, m, d_in) or W0.dtype != torch.float32 or W0.device != x.device
            or not W0.is_contiguous()):
        raise ValueError(f"W0 must be a contiguous float32 [H, {m}, d_in] tensor on x's device")
    if chunk_steps < 0:
        raise ValueError("chunk_steps must be >= 0")
    W_T = (torch.empty((B, H, m, d_in), dtype=torch.float32, device=x.device)
           if return_state or overlap else None)
    aux = aux_obj = None
    if overlap:
        aux_obj = aux_stream if aux_stream is not None else _aux_stream(x.device)
        aux = _stream_handle(x, aux_obj)
    main = stream if stream is not None else torch.cuda.current_stream(x.device)
    _check_aligned(x=x, W0=W0, F0=F0, z=z, y=y)
    a = _lib.SrdeltanetArgs(x=_ptr(x), W0=_ptr(W0), F0=_ptr(F0), z=_ptr(z), y=_ptr(y), W_T=_ptr(W_T),
                            F_T=_ptr(F_T), B=B, T=T, H=H, d_in=d_in, d_key=d_key, d_v=d_v, n_lr=int(n_lr),
                            apply_input_softmax=int(bool(apply_input_softmax)),
                            stream=_stream_handle(x, stream), aux_stream=aux, chunk_steps=int(chunk_steps))
    with torch.cuda.device(x.device):
        rc = lib.srwm_srdeltanet_forward(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    if not return_state:
        # the chunks' carried states, read and rewritten by kernels on both streams
        _hold_for(W_T, x.device, main, aux_obj)
        _hold_for(F_T, x.device, main, aux_obj)
        W_T = F_T = None
    return y, W_T, F_T, z


def deltanet_project(x, W_slow, d_key: int, d_v: int, z=None, stream=None):
    """DeltaNet's slow projection alone: z [B, T, H, P] for every step."""
    import torch

    lib = _lib.load()
    B, T, H, d_in, P, z, _, _ = _fwp_common(x, None, d_key, d_v, False, z, None)
    if (tuple(W_slow.shape) != (H * P, H * d_in) or W_slow.dtype != torch.float32
            or W_slow.device != x.device or not W_slow.is_contiguous()):
        raise ValueError("W_slow must be a contiguous float32 [H*P, H*d_in] tensor on x's device")
    _check_aligned(x=x, W_slow=W_slow, z=z)
    a = _lib.DeltanetArgs(x=_ptr(x), W_slow=_ptr(W_slow), F0=None, z=_ptr(z), y=None, F_T=None,
                          B=B, T=T, H=H, d_in=d_in, d_key=d_key, d_v=d_v, stream=_stream_handle(x, stream))
    with torch.cuda.device(x.device):
        rc = lib.srwm_deltanet_project(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    return z


def srdeltanet_chunk_steps(B: int, T: int, H: int, d_in: int, d_key: int, d_v: int, n_lr: int = 4) -> int:
    """Steps per chunk of srdeltanet_forward's overlapped schedule for these
    sizes (T: the halves run one after the other)."""
    c = _lib.load().srwm_srdeltanet_chunk_steps(B, T, H, d_in, d_key, d_v, n_lr)
    if c < 0:
        raise ValueError(_lib.strerror(int(c)))
    return int(c)


def fast_forward(z, d_key: int, d_v: int, F0=None, return_state: bool = False, y=None, stream=None, F_T=None):
    """The fast-matrix recurrence alone from given projections z [B, T, H, P]:
    returns (y [B, T, H, d_v], F_T or None).  ``z`` and ``y`` may be the same
    time slice [:, t0:t1] of longer [B, S, H, *] buffers; ``F_T`` may be
    passed preallocated (then it is returned)."""
    import torch

    lib = _lib.load()
    if not isinstance(z, torch.Tensor) or z.device.type != "cuda" or z.dtype != torch.float32 \
            or z.dim() != 4 or z.shape[-1] != d_v + 2 * d_key + 1:
        raise ValueError("z must be a float32 [B, T, H, d_v + 2*d_key + 1] tensor on a ROCm GPU")
    t_stride = _time_stride(z, "z")
    B, T, H, _ = z.shape
    if F0 is not None and (tuple(F0.shape) != (B, H, d_v, d_key) or F0.dtype != torch.float32
                           or F0.device != z.device or not F0.is_contiguous()):
        raise ValueError("F0 must be a contiguous float32 [B, H, d_v, d_key] tensor on z's device")
    if y is None:
        if t_stride:
            raise ValueError("z is a time slice of longer sequences: pass y, a slice of the same steps")
        y = torch.empty((B, T, H, d_v), dtype=torch.float32, device=z.device)
    elif (tuple(y.shape) != (B, T, H, d_v) or y.dtype != torch.float32 or y.device != z.device
          or _time_stride(y, "y") != t_stride):
        raise ValueError("y must be a float32 [B, T, H, d_v] tensor laid out like z")
    if F_T is not None:
        if (tuple(F_T.shape) != (B, H, d_v, d_key) or F_T.dtype != torch.float32 or F_T.device != z.device
                or not F_T.is_contiguous()):
            raise ValueError("F_T must be a contiguous float32 [B, H, d_v, d_key] tensor on z's device")
    elif return_state:
        F_T = torch.empty((B, H, d_v, d_key), dtype=torch.float32, device=z.device)
    _check_aligned(F0=F0, y=y, F_T=F_T)  # z's rows are read at any offset
    a = _lib.FastArgs(z=_ptr(z), F0=_ptr(F0), y=_ptr(y), F_T=_ptr(F_T), B=B, T=T, H=H, d_key=d_key, d_v=d_v,
                      stream=_stream_handle(z, stream), t_stride=t_stride)
    with torch.cuda.device(z.device):
        rc = lib.srwm_fast_forward(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    return y, F_T
