"""Comparison rules between the GPU path and the float64 oracle.

Tolerances (fp32 state in every case):
  * fp32 I/O: relative L2 <= 2e-4 on y and on W_T, and max|dy| <= 1e-3 * max|y|.
  * gradients (float32 backward against the float64 gradient oracle):
    relative L2 <= 1e-4 on dx and dW0, and max|d| <= 1e-3 * max|ref|.  The
    same recurrence differentiated by autograd in float32 instead of float64
    drifts by 5e-7 .. 1e-6 (relative L2, T = 512); 1e-4 leaves two orders of
    magnitude for the backward's different summation order and for undoing
    each update by subtraction.
  * bf16 I/O: relative L2 <= 1e-2 on y.  The max-abs clause is applied against
    the oracle's y rounded to bf16 with one bf16 ulp of headroom per element,
    |dy_i| <= 1e-3 * max|y| + ulp_bf16(y_i): bf16 output rounding alone can err
    by half an ulp (~2e-3 relative), which the literal clause would not allow.
"""
from __future__ import annotations

import numpy as np

from self_referential_weight_amd.workloads import round_to_bf16

RTOL_L2_F32 = 2e-4
RTOL_L2_BF16 = 1e-2
MAXABS_FRAC = 1e-3
RTOL_L2_GRAD = 1e-4


def rel_l2(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((a - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def ulp_bf16(v):
    v = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(v, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_y(y_gpu, y_ref, io_dtype, what=""):
    y_gpu = np.asarray(y_gpu, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    ymax = float(np.abs(y_ref).max()) if y_ref.size else 0.0
    r = rel_l2(y_gpu, y_ref)
    if io_dtype == "bf16":
        assert r <= RTOL_L2_BF16, f"{what} y relL2 {r:.3e}"
        yb = round_to_bf16(y_ref.astype(np.float32)).astype(np.float64)
        bound = MAXABS_FRAC * ymax + ulp_bf16(y_ref)
        bad = np.abs(y_gpu - yb) > bound
        assert not bad.any(), f"{what} {int(bad.sum())} bf16 outputs beyond 1e-3*max|y| + 1 ulp"
    else:
        assert r <= RTOL_L2_F32, f"{what} y relL2 {r:.3e}"
        d = float(np.abs(y_gpu - y_ref).max()) if y_ref.size else 0.0
        assert d <= MAXABS_FRAC * ymax, f"{what} y max-abs {d:.3e} vs max|y| {ymax:.3e}"
    return r


def check_state(W_gpu, W_ref, what=""):
    r = rel_l2(W_gpu, W_ref)
    assert r <= RTOL_L2_F32, f"{what} W_T relL2 {r:.3e}"
    d = float(np.abs(np.asarray(W_gpu, np.float64) - W_ref).max())
    assert d <= MAXABS_FRAC * float(np.abs(W_ref).max()), f"{what} W_T max-abs {d:.3e}"
    return r


def check_grad(g_gpu, g_ref, what="", rtol=RTOL_L2_GRAD):
    g_gpu = np.asarray(g_gpu, np.float64)
    g_ref = np.asarray(g_ref, np.float64)
    if g_ref.size == 0:
        assert g_gpu.size == 0
        return 0.0
    r = rel_l2(g_gpu, g_ref)
    assert r <= rtol, f"{what} relL2 {r:.3e}"
    d = float(np.abs(g_gpu - g_ref).max())
    assert d <= MAXABS_FRAC * float(np.abs(g_ref).max()), f"{what} max-abs {d:.3e}"
    return r
