"""ctypes view of libsrwm.so (declarations in include/srwm.h)."""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsrwm.so"

SRWM_IO_F32 = 0
SRWM_IO_BF16 = 1

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(
            f"libsrwm is not built ({LIB_PATH} missing); run __graft_entry__.build() "
            "or python -m self_referential_weight_amd._build")
    lib = ctypes.CDLL(str(LIB_PATH))
    i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    fwd_args = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, ci, vp]
    lib.srwm_forward.argtypes = fwd_args
    lib.srwm_forward.restype = ci
    lib.srwm_forward_variant.argtypes = fwd_args + [ci]
    lib.srwm_forward_variant.restype = ci
    lib.srwm_variant_count.argtypes = []
    lib.srwm_variant_count.restype = ci
    ip = ctypes.POINTER(ci)
    lib.srwm_variant_info.argtypes = [ci, ip, ip, ip, ip, ip, ip, ip, ip]
    lib.srwm_variant_info.restype = ci
    lib.srwm_select_variant.argtypes = [i64, i64, ci, i64]
    lib.srwm_select_variant.restype = ci
    lib.srwm_supported.argtypes = [i64, i64, ci]
    lib.srwm_supported.restype = ci
    lib.srwm_strerror.argtypes = [ci]
    lib.srwm_strerror.restype = ctypes.c_char_p
    lib.srwm_version.argtypes = []
    lib.srwm_version.restype = ci
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().srwm_strerror(int(code)).decode()


def variants() -> list[dict]:
    lib = load()
    out = []
    for i in range(lib.srwm_variant_count()):
        vals = [ctypes.c_int() for _ in range(8)]
        rc = lib.srwm_variant_info(i, *[ctypes.byref(v) for v in vals])
        assert rc == 0
        d_in, d_out, io, nw, p, wpe, sched, auto = (v.value for v in vals)
        out.append(dict(index=i, d_in=d_in, d_out=d_out,
                        io_dtype="bf16" if io == SRWM_IO_BF16 else "f32",
                        waves=nw, lanes_per_row=p, waves_per_simd=wpe,
                        schedule="fused" if sched else "phased", auto=bool(auto)))
    return out
