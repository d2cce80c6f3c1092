"""ctypes view of libsrwm.so (declarations in include/srwm.h)."""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libsrwm.so"

SRWM_IO_F32 = 0
SRWM_IO_BF16 = 1


class ForwardArgs(ctypes.Structure):
    """srwm_forward_args_t."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("W0", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("W_T", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_out", ctypes.c_int64),
        ("m", ctypes.c_int64),
        ("io_dtype", ctypes.c_int),
        ("apply_input_softmax", ctypes.c_int),
        ("n_lr", ctypes.c_int),
        ("w0_per_sequence", ctypes.c_int),
        ("reset_interval", ctypes.c_int64),
        ("variant", ctypes.c_int),
        ("stream", ctypes.c_void_p),
        ("tape", ctypes.c_void_p),
        ("window_states", ctypes.c_void_p),
        ("t_stride", ctypes.c_int64),
    ]


class BackwardArgs(ctypes.Structure):
    """srwm_backward_args_t."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("W_T", ctypes.c_void_p),
        ("tape", ctypes.c_void_p),
        ("gy", ctypes.c_void_p),
        ("gW_T", ctypes.c_void_p),
        ("dx", ctypes.c_void_p),
        ("dW_init", ctypes.c_void_p),
        ("dW0", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_out", ctypes.c_int64),
        ("m", ctypes.c_int64),
        ("io_dtype", ctypes.c_int),
        ("apply_input_softmax", ctypes.c_int),
        ("n_lr", ctypes.c_int),
        ("stream", ctypes.c_void_p),
        ("reset_interval", ctypes.c_int64),
        ("window_states", ctypes.c_void_p),
    ]


class DeltanetArgs(ctypes.Structure):
    """srwm_deltanet_args_t."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("W_slow", ctypes.c_void_p),
        ("F0", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("F_T", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_key", ctypes.c_int64),
        ("d_v", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
    ]


class SrdeltanetArgs(ctypes.Structure):
    """srwm_srdeltanet_args_t."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("W0", ctypes.c_void_p),
        ("F0", ctypes.c_void_p),
        ("z", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("W_T", ctypes.c_void_p),
        ("F_T", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("d_key", ctypes.c_int64),
        ("d_v", ctypes.c_int64),
        ("n_lr", ctypes.c_int),
        ("apply_input_softmax", ctypes.c_int),
        ("stream", ctypes.c_void_p),
        ("aux_stream", ctypes.c_void_p),
        ("chunk_steps", ctypes.c_int64),
    ]


class FastArgs(ctypes.Structure):
    """srwm_fast_args_t."""
    _fields_ = [
        ("z", ctypes.c_void_p),
        ("F0", ctypes.c_void_p),
        ("y", ctypes.c_void_p),
        ("F_T", ctypes.c_void_p),
        ("B", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("d_key", ctypes.c_int64),
        ("d_v", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
        ("t_stride", ctypes.c_int64),
    ]


class VariantInfo(ctypes.Structure):
    """srwm_variant_info_t."""
    _fields_ = [(name, ctypes.c_int) for name in (
        "d_in", "d_out", "io_dtype", "n_lr", "waves", "lanes_per_row", "waves_per_simd",
        "schedule", "supports_reset", "writes_tape", "is_auto")]


class KernelResources(ctypes.Structure):
    """srwm_kernel_resources_t."""
    _fields_ = [(name, ctypes.c_int) for name in (
        "vgprs", "lds_bytes", "scratch_bytes", "threads", "workgroups_per_cu", "waves_per_simd")]


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
    lib.srwm_forward_ex.argtypes = [ctypes.POINTER(ForwardArgs)]
    lib.srwm_forward_ex.restype = ci
    lib.srwm_backward.argtypes = [ctypes.POINTER(BackwardArgs)]
    lib.srwm_backward.restype = ci
    lib.srwm_backward_noalloc.argtypes = [ctypes.POINTER(BackwardArgs)]
    lib.srwm_backward_noalloc.restype = ci
    lib.srwm_backward_noalloc_scratch_bytes.argtypes = []
    lib.srwm_backward_noalloc_scratch_bytes.restype = i64
    lib.srwm_tape_row.argtypes = [i64, i64, ci]
    lib.srwm_tape_row.restype = i64
    lib.srwm_backward_supported.argtypes = [i64, i64, ci, ci]
    lib.srwm_backward_supported.restype = ci
    lib.srwm_deltanet_forward.argtypes = [ctypes.POINTER(DeltanetArgs)]
    lib.srwm_deltanet_forward.restype = ci
    lib.srwm_srdeltanet_forward.argtypes = [ctypes.POINTER(SrdeltanetArgs)]
    lib.srwm_srdeltanet_forward.restype = ci
    lib.srwm_deltanet_project.argtypes = [ctypes.POINTER(DeltanetArgs)]
    lib.srwm_deltanet_project.restype = ci
    lib.srwm_fast_forward.argtypes = [ctypes.POINTER(FastArgs)]
    lib.srwm_fast_forward.restype = ci
    lib.srwm_fwp_supported.argtypes = [i64, i64]
    lib.srwm_fwp_supported.restype = ci
    lib.srwm_srdeltanet_chunk_steps.argtypes = [i64, i64, i64, i64, i64, i64, ci]
    lib.srwm_srdeltanet_chunk_steps.restype = i64
    lib.srwm_valu_probe.argtypes = [ctypes.c_void_p, i64, ci, ctypes.c_void_p]
    lib.srwm_valu_probe.restype = ci
    lib.srwm_valu_probe_flop.argtypes = [i64, ci]
    lib.srwm_valu_probe_flop.restype = i64
    lib.srwm_lds_probe.argtypes = [ctypes.c_void_p, i64, ci, ctypes.c_void_p]
    lib.srwm_lds_probe.restype = ci
    lib.srwm_lds_probe_bytes.argtypes = [i64, ci]
    lib.srwm_lds_probe_bytes.restype = i64
    lib.srwm_variant_count.argtypes = []
    lib.srwm_variant_count.restype = ci
    lib.srwm_variant_info.argtypes = [ci, ctypes.POINTER(VariantInfo)]
    lib.srwm_variant_info.restype = ci
    lib.srwm_variant_resources.argtypes = [ci, ctypes.POINTER(KernelResources)]
    lib.srwm_variant_resources.restype = ci
    lib.srwm_backward_resources.argtypes = [i64, i64, ci, ci, i64, ctypes.POINTER(KernelResources)]
    lib.srwm_backward_resources.restype = ci
    lib.srwm_select_variant.argtypes = [i64, i64, ci, ci, i64, i64]
    lib.srwm_select_variant.restype = ci
    lib.srwm_supported.argtypes = [i64, i64, ci, ci]
    lib.srwm_supported.restype = ci
    lib.srwm_strerror.argtypes = [ci]
    lib.srwm_strerror.restype = ctypes.c_char_p
    lib.srwm_version.argtypes = []
    lib.srwm_version.restype = ci
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().srwm_strerror(int(code)).decode()


def _resources(rc: int, r: KernelResources) -> dict:
    if rc != 0:
        raise RuntimeError(strerror(rc))
    return {name: getattr(r, name) for name, _ in KernelResources._fields_}


def variant_resources(i: int) -> dict:
    r = KernelResources()
    return _resources(load().srwm_variant_resources(int(i), ctypes.byref(r)), r)


def backward_resources(d_in: int, d_out: int, n_lr: int = 4, reset: bool = False, units: int = 2048) -> dict:
    r = KernelResources()
    return _resources(load().srwm_backward_resources(int(d_in), int(d_out), int(n_lr), int(bool(reset)),
                                                     int(units), ctypes.byref(r)), r)


def variants() -> list[dict]:
    lib = load()
    out = []
    for i in range(lib.srwm_variant_count()):
        info = VariantInfo()
        rc = lib.srwm_variant_info(i, ctypes.byref(info))
        assert rc == 0
        out.append(dict(index=i, d_in=info.d_in, d_out=info.d_out,
                        io_dtype="bf16" if info.io_dtype == SRWM_IO_BF16 else "f32",
                        n_lr=info.n_lr, waves=info.waves, lanes_per_row=info.lanes_per_row,
                        waves_per_simd=info.waves_per_simd,
                        schedule="fused" if info.schedule else "phased",
                        supports_reset=bool(info.supports_reset),
                        writes_tape=bool(info.writes_tape), auto=bool(info.is_auto)))
    return out
