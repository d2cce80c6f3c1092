"""Python access to the float64 SRWM oracle (oracle/srwm_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``self_referential_weight_amd``) never imports it and has no CPU fallback.

The C file holds every formula and cites the pages for each step; this module
only marshals numpy arrays in and out, and builds the shared library with gcc
(``-O2 -ffp-contract=off``, no fast-math, no BLAS).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "srwm_oracle.c"
_LIB = _HERE / "libsrwm_oracle.so"

_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-std=c11", "-Wall"]


def build(force: bool = False) -> Path:
    """Compile the oracle (float64 and the float32 study variant) with gcc."""
    if not force and _LIB.exists() and _LIB.stat().st_mtime >= _SRC.stat().st_mtime:
        return _LIB
    tmp = _LIB.with_suffix(".so.tmp")
    objs = []
    for tag, extra in (("f64", []), ("f32", ["-DORACLE_FLOAT"])):
        obj = _HERE / f"_srwm_oracle_{tag}.o"
        subprocess.check_call(["gcc", *_CFLAGS, *extra, "-c", str(_SRC), "-o", str(obj)])
        objs.append(str(obj))
    subprocess.check_call(["gcc", "-shared", "-o", str(tmp), *objs, "-lm", "-lpthread"])
    os.replace(tmp, _LIB)
    for o in objs:
        os.unlink(o)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(str(_LIB))
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        for prefix, p in (("srwm_oracle_", dp), ("srwm_oracle_f32_", fp)):
            f = getattr(lib, prefix + "delta_update")
            f.argtypes = [p, ctypes.c_int, ctypes.c_int, p, p, p, p, p]
            f.restype = None
            f = getattr(lib, prefix + "step")
            f.argtypes = [p, ctypes.c_int, ctypes.c_int, ctypes.c_int, p, ctypes.c_int] + [p] * 8
            f.restype = None
            f = getattr(lib, prefix + "forward")
            f.argtypes = [p, p, p, p, ctypes.c_long, ctypes.c_long, ctypes.c_long,
                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                          ctypes.c_long, ctypes.c_int]
            f.restype = ctypes.c_int
            f = getattr(lib, prefix + "fast_step")
            f.argtypes = [p, ctypes.c_int, ctypes.c_int, p, p, p, p, p, p]
            f.restype = None
            L = ctypes.c_long
            f = getattr(lib, prefix + "deltanet_forward")
            f.argtypes = [p, p, p, p, p, L, L, L, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
            f.restype = ctypes.c_int
            f = getattr(lib, prefix + "srdeltanet_forward")
            f.argtypes = [p, p, p, p, p, p, L, L, L] + [ctypes.c_int] * 6
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray | None, ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    """Worker threads: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when set and at 16 (one GPU's share of a host)."""
    try:
        n = max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return min(n, 16)


def m_rows(d_in: int, d_out: int, n_lr: int = 4) -> int:
    return d_out + 2 * d_in + n_lr


def delta_update(W, kh, qh, eta):
    """Given-address delta update.  Returns (W_new, v, vb)."""
    lib = _load()
    W = np.array(W, dtype=np.float64, order="C", copy=True)
    rows, d_in = W.shape
    kh = np.ascontiguousarray(kh, dtype=np.float64)
    qh = np.ascontiguousarray(qh, dtype=np.float64)
    eta = np.ascontiguousarray(np.broadcast_to(np.asarray(eta, np.float64), (rows,)))
    v = np.empty(rows)
    vb = np.empty(rows)
    d = ctypes.c_double
    lib.srwm_oracle_delta_update(_ptr(W, d), rows, d_in, _ptr(kh, d), _ptr(qh, d),
                                 _ptr(eta, d), _ptr(v, d), _ptr(vb, d))
    return W, v, vb


def step(W, x_t, d_out: int, apply_input_softmax: bool, n_lr: int = 4):
    """One step on one unit.  Returns a dict with W (= W_t), y, u, z, kh, qh, g, v, vb."""
    lib = _load()
    W = np.array(W, dtype=np.float64, order="C", copy=True)
    m, d_in = W.shape
    assert m == m_rows(d_in, d_out, n_lr)
    x_t = np.ascontiguousarray(x_t, dtype=np.float64)
    out = {k: np.empty(n) for k, n in (("y", d_out), ("u", d_in), ("z", m), ("kh", d_in),
                                       ("qh", d_in), ("g", n_lr), ("v", m), ("vb", m))}
    d = ctypes.c_double
    lib.srwm_oracle_step(_ptr(W, d), d_in, d_out, n_lr, _ptr(x_t, d), int(bool(apply_input_softmax)),
                         *[_ptr(out[k], d) for k in ("y", "u", "z", "kh", "qh", "g", "v", "vb")])
    out["W"] = W
    return out


def _forward(prefix, npdtype, ctype, x, W0, apply_input_softmax, return_state, nthreads,
             n_lr, reset_interval):
    lib = _load()
    x = np.ascontiguousarray(x, dtype=npdtype)
    W0 = np.ascontiguousarray(W0, dtype=npdtype)
    B, T, H, d_in = x.shape
    per_seq = W0.ndim == 4
    if per_seq:
        B2, H2, m, d_in2 = W0.shape
        assert B2 == B
    else:
        H2, m, d_in2 = W0.shape
    assert H2 == H and d_in2 == d_in
    d_out = m - 2 * d_in - n_lr
    assert d_out >= 1
    y = np.empty((B, T, H, d_out), dtype=npdtype)
    WT = np.empty((B, H, m, d_in), dtype=npdtype) if return_state else None
    n = default_threads() if nthreads is None else int(nthreads)
    rc = getattr(lib, prefix + "forward")(_ptr(x, ctype), _ptr(W0, ctype), _ptr(y, ctype),
                                          _ptr(WT, ctype), B, T, H, d_in, d_out, int(n_lr),
                                          int(bool(apply_input_softmax)), int(per_seq),
                                          int(reset_interval), n)
    if rc != 0:
        raise ValueError(f"oracle forward rejected its arguments (code {rc})")
    return y, WT


def forward(x, W0, apply_input_softmax=False, return_state=True, nthreads=None, n_lr=4,
            reset_interval=0):
    """float64 oracle: x[B,T,H,d_in], W0[H,m,d_in] (shared) or W0[B,H,m,d_in]
    (per sequence) -> (y[B,T,H,d_out], W_T[B,H,m,d_in]).  m = d_out+2*d_in+n_lr;
    reset_interval R > 0 returns the state to W0 before every step t>0, t%R==0."""
    return _forward("srwm_oracle_", np.float64, ctypes.c_double, x, W0,
                    apply_input_softmax, return_state, nthreads, n_lr, reset_interval)


def forward_f32(x, W0, apply_input_softmax=False, return_state=True, nthreads=None, n_lr=4,
                reset_interval=0):
    """The same definition evaluated in float32 (drift study only)."""
    return _forward("srwm_oracle_f32_", np.float32, ctypes.c_float, x, W0,
                    apply_input_softmax, return_state, nthreads, n_lr, reset_interval)


# ---------------------------------------------------------------------------
# DeltaNet / SR-DeltaNet (the C file states the definitions and their sources).
def proj_rows(d_key: int, d_v: int) -> int:
    """Rows of one head's projection [k; v; q; beta]: d_v + 2*d_key + 1."""
    return d_v + 2 * d_key + 1


def fast_step(F, p, d_key: int, d_v: int):
    """One fast-matrix step.  Returns a dict with F (updated), y, kh, qh, g, vb."""
    lib = _load()
    F = np.array(F, dtype=np.float64, order="C", copy=True)
    assert F.shape == (d_v, d_key)
    p = np.ascontiguousarray(p, dtype=np.float64)
    assert p.shape == (proj_rows(d_key, d_v),)
    out = {k: np.empty(n) for k, n in (("y", d_v), ("kh", d_key), ("qh", d_key), ("g", 1), ("vb", d_v))}
    d = ctypes.c_double
    lib.srwm_oracle_fast_step(_ptr(F, d), d_key, d_v, _ptr(p, d),
                              *[_ptr(out[k], d) for k in ("y", "kh", "qh", "g", "vb")])
    out["F"] = F
    return out


def deltanet_forward(x, Wslow, d_key: int, d_v: int, F0=None, nthreads=None, f32=False):
    """x[B,T,H,d_in], Wslow[H*P, H*d_in] -> (y[B,T,H,d_v], F_T[B,H,d_v,d_key]);
    F0: None (zero) or [B,H,d_v,d_key].  f32=True evaluates the same definition
    in float32 (drift study only)."""
    lib = _load()
    dt, d, fn = ((np.float32, ctypes.c_float, lib.srwm_oracle_f32_deltanet_forward) if f32 else
                 (np.float64, ctypes.c_double, lib.srwm_oracle_deltanet_forward))
    x = np.ascontiguousarray(x, dtype=dt)
    B, T, H, d_in = x.shape
    P = proj_rows(d_key, d_v)
    Wslow = np.ascontiguousarray(Wslow, dtype=dt)
    assert Wslow.shape == (H * P, H * d_in)
    if F0 is not None:
        F0 = np.ascontiguousarray(F0, dtype=dt)
        assert F0.shape == (B, H, d_v, d_key)
    y = np.empty((B, T, H, d_v), dtype=dt)
    FT = np.empty((B, H, d_v, d_key), dtype=dt)
    n = default_threads() if nthreads is None else int(nthreads)
    rc = fn(_ptr(x, d), _ptr(Wslow, d), _ptr(F0, d), _ptr(y, d), _ptr(FT, d), B, T, H, d_in, d_key, d_v, n)
    if rc != 0:
        raise ValueError(f"oracle deltanet_forward rejected its arguments (code {rc})")
    return y, FT


def srdeltanet_forward(x, W0, d_key: int, d_v: int, F0=None, apply_input_softmax=False, n_lr=4,
                       nthreads=None):
    """x[B,T,H,d_in], SRWM W0[H,m,d_in] (m = P + 2*d_in + n_lr) ->
    (y[B,T,H,d_v], W_T[B,H,m,d_in], F_T[B,H,d_v,d_key])."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, T, H, d_in = x.shape
    P = proj_rows(d_key, d_v)
    W0 = np.ascontiguousarray(W0, dtype=np.float64)
    m = P + 2 * d_in + n_lr
    assert W0.shape == (H, m, d_in)
    if F0 is not None:
        F0 = np.ascontiguousarray(F0, dtype=np.float64)
        assert F0.shape == (B, H, d_v, d_key)
    y = np.empty((B, T, H, d_v))
    WT = np.empty((B, H, m, d_in))
    FT = np.empty((B, H, d_v, d_key))
    n = default_threads() if nthreads is None else int(nthreads)
    d = ctypes.c_double
    rc = lib.srwm_oracle_srdeltanet_forward(_ptr(x, d), _ptr(W0, d), _ptr(F0, d), _ptr(y, d), _ptr(WT, d),
                                            _ptr(FT, d), B, T, H, d_in, d_key, d_v, int(n_lr),
                                            int(bool(apply_input_softmax)), n)
    if rc != 0:
        raise ValueError(f"oracle srdeltanet_forward rejected its arguments (code {rc})")
    return y, WT, FT
