"""MI355X-native forward recurrence of the multi-head, 4-learning-rate
self-referential weight matrix (SRWM).

``forward`` is a thin binding over ``srwm_forward`` of libsrwm (include/srwm.h):
it checks and marshals torch device tensors and the current HIP stream; every
step of the recurrence runs in the library's HIP kernels.  There is no CPU or
PyTorch fallback: without the built library, or with tensors off the GPU, the
call raises.
"""
from __future__ import annotations

from . import _lib
from .workloads import HEADLINE, WORKLOADS, Workload

__all__ = ["forward", "supported", "variants", "select_variant", "m_rows", "WORKLOADS", "HEADLINE", "Workload"]


def m_rows(d_in: int, d_out: int, n_lr: int = 4) -> int:
    """Rows of the state: d_out + 2*d_in + n_lr (y, k, q blocks and the rate logits)."""
    return d_out + 2 * d_in + n_lr


def _io(io_dtype: str) -> int:
    return _lib.SRWM_IO_BF16 if io_dtype == "bf16" else _lib.SRWM_IO_F32


def supported(d_in: int, d_out: int, io_dtype: str = "f32", n_lr: int = 4) -> bool:
    return bool(_lib.load().srwm_supported(d_in, d_out, _io(io_dtype), n_lr))


def variants() -> list[dict]:
    return _lib.variants()


def select_variant(d_in: int, d_out: int, io_dtype: str, units: int, n_lr: int = 4,
                   reset_interval: int = 0) -> dict:
    """The kernel variant the automatic choice uses for B*H = units."""
    i = _lib.load().srwm_select_variant(d_in, d_out, _io(io_dtype), n_lr, reset_interval, units)
    if i < 0:
        raise RuntimeError(_lib.strerror(i))
    return _lib.variants()[i]


def forward(x, W0, apply_input_softmax: bool = False, return_state: bool = False,
            variant: int = -1, y=None, W_T=None, stream=None, n_lr: int = 4,
            reset_interval: int = 0):
    """Run the SRWM recurrence on the GPU.

    x   : torch tensor [B, T, H, d_in], float32 or bfloat16, on a ROCm device
    W0  : torch float32 tensor [H, m, d_in] (shared over the batch) or
          [B, H, m, d_in] (one initial state per sequence, e.g. an earlier
          W_T), m = d_out + 2*d_in + n_lr, same device
    n_lr: 4 (a learning rate per row block) or 1 (one for every row)
    reset_interval: 0, or R > 0 to return every state to W0 before each step
          t > 0 with t % R == 0 (the reset ablation)
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
    if not (x.is_contiguous() and W0.is_contiguous()):
        raise ValueError("x and W0 must be contiguous")
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
        y = torch.empty((B, T, H, d_out), dtype=x.dtype, device=x.device)
    elif (tuple(y.shape) != (B, T, H, d_out) or y.dtype != x.dtype or y.device != x.device
          or not y.is_contiguous()):
        raise ValueError("preallocated y has the wrong shape/dtype/device/layout")
    if return_state:
        if W_T is None:
            W_T = torch.empty((B, H, m, d_in), dtype=torch.float32, device=x.device)
        elif (tuple(W_T.shape) != (B, H, m, d_in) or W_T.dtype != torch.float32
              or W_T.device != x.device or not W_T.is_contiguous()):
            raise ValueError("preallocated W_T has the wrong shape/dtype/device/layout")
    else:
        W_T = None
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
        stream=handle)
    with torch.cuda.device(x.device):
        rc = lib.srwm_forward_ex(a)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    return y, W_T
