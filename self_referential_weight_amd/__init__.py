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


def m_rows(d_in: int, d_out: int) -> int:
    """Rows of the state: d_out + 2*d_in + 4 (y, k, q blocks and 4 rate logits)."""
    return d_out + 2 * d_in + 4


def supported(d_in: int, d_out: int, io_dtype: str = "f32") -> bool:
    io = _lib.SRWM_IO_BF16 if io_dtype == "bf16" else _lib.SRWM_IO_F32
    return bool(_lib.load().srwm_supported(d_in, d_out, io))


def variants() -> list[dict]:
    return _lib.variants()


def select_variant(d_in: int, d_out: int, io_dtype: str, units: int) -> dict:
    """The kernel variant the automatic choice uses for B*H = units."""
    io = _lib.SRWM_IO_BF16 if io_dtype == "bf16" else _lib.SRWM_IO_F32
    i = _lib.load().srwm_select_variant(d_in, d_out, io, units)
    if i < 0:
        raise RuntimeError(_lib.strerror(i))
    return _lib.variants()[i]


def forward(x, W0, apply_input_softmax: bool = False, return_state: bool = False,
            variant: int = -1, y=None, W_T=None, stream=None):
    """Run the SRWM recurrence on the GPU.

    x   : torch tensor [B, T, H, d_in], float32 or bfloat16, on a ROCm device
    W0  : torch float32 tensor [H, m, d_in], m = d_out + 2*d_in + 4, same device
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
    if x.dim() != 4 or W0.dim() != 3:
        raise ValueError("x must be [B,T,H,d_in] and W0 [H,m,d_in]")
    if not (x.is_contiguous() and W0.is_contiguous()):
        raise ValueError("x and W0 must be contiguous")
    B, T, H, d_in = x.shape
    H2, m, d_in2 = W0.shape
    if H2 != H or d_in2 != d_in:
        raise ValueError(f"W0 shape {tuple(W0.shape)} does not match x {tuple(x.shape)}")
    d_out = m - 2 * d_in - 4
    if d_out < 1:
        raise ValueError(f"W0 has {m} rows; need d_out + 2*d_in + 4 with d_out >= 1")
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
    with torch.cuda.device(x.device):
        rc = lib.srwm_forward_variant(
            x.data_ptr() if x.numel() else None, W0.data_ptr() if W0.numel() else None,
            y.data_ptr() if y.numel() else None, W_T.data_ptr() if W_T is not None and W_T.numel() else None,
            B, T, H, d_in, d_out, m, io, int(bool(apply_input_softmax)), handle, int(variant))
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    return y, W_T
