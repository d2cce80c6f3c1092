"""The C ABI of libsrwm without a GPU: every symbol include/srwm.h declares is
exported, and invalid calls are rejected by validation before any HIP call."""
import ctypes
import re
from pathlib import Path

import pytest

from self_referential_weight_amd import _lib

HEADER = Path(__file__).resolve().parents[1] / "include" / "srwm.h"

OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIAS, E_HIP, E_ARG, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(srwm_\w+)\s*\(", text)))


def test_header_symbols_exported():
    lib = _lib.load()
    names = declared_functions()
    assert {"srwm_forward", "srwm_strerror", "srwm_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    lib = _lib.load()
    assert lib.srwm_version() == 800
    for code in (OK, E_NULL, E_SHAPE, E_UNSUP, E_ALIAS, E_HIP, E_ARG, E_SCRATCH):
        assert _lib.strerror(code).startswith("SRWM_")
    assert "unknown" in _lib.strerror(-99)


def test_variant_table_covers_workloads():
    from self_referential_weight_amd.workloads import WORKLOADS
    vs = _lib.variants()
    assert len(vs) == _lib.load().srwm_variant_count()
    for w in WORKLOADS.values():
        io = _lib.SRWM_IO_BF16 if w.io_dtype == "bf16" else _lib.SRWM_IO_F32
        assert _lib.load().srwm_supported(w.d_in, w.d_out, io, 4) == 1, w.name
        assert _lib.load().srwm_supported(w.d_in, w.d_out, io, 1) == 1, w.name
    # every supported shape has an automatically eligible variant, and one that
    # implements the reset ablation
    shapes = {(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) for v in vs}
    auto = {(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) for v in vs if v["auto"]}
    reset = {(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) for v in vs if v["supports_reset"]}
    assert shapes == auto == reset
    info = _lib.VariantInfo()
    assert _lib.load().srwm_variant_info(len(vs), ctypes.byref(info)) == E_ARG
    assert _lib.load().srwm_variant_info(0, None) == E_NULL


FAKE_X, FAKE_W0, FAKE_Y, FAKE_WT = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def call(x=FAKE_X, W0=FAKE_W0, y=FAKE_Y, WT=FAKE_WT, B=2, T=3, H=2, d_in=16, d_out=16,
         m=None, io=0, flag=0, variant=None):
    lib = _lib.load()
    m = d_out + 2 * d_in + 4 if m is None else m
    args = (x, W0, y, WT, B, T, H, d_in, d_out, m, io, flag, None)
    if variant is None:
        return lib.srwm_forward(*args)
    return lib.srwm_forward_variant(*args, variant)


@pytest.mark.parametrize("kw,code", [
    (dict(m=51), E_SHAPE),
    (dict(B=-1), E_SHAPE),
    (dict(T=-5), E_SHAPE),
    (dict(H=-1), E_SHAPE),
    (dict(d_in=0), E_SHAPE),
    (dict(d_out=0, m=36), E_SHAPE),
    (dict(d_in=7, d_out=7), E_UNSUP),
    (dict(d_in=64, d_out=32), E_UNSUP),
    (dict(io=2), E_ARG),
    (dict(flag=2), E_ARG),
    (dict(variant=-2), E_ARG),
    (dict(variant=10 ** 6), E_ARG),
    (dict(x=None), E_NULL),
    (dict(y=None), E_NULL),
    (dict(W0=None), E_NULL),
    (dict(y=FAKE_X), E_ALIAS),
    (dict(y=FAKE_X + 64), E_ALIAS),
    (dict(WT=FAKE_W0), E_ALIAS),
    (dict(WT=FAKE_Y + 16), E_ALIAS),
    (dict(B=2 ** 40, T=2 ** 40), E_SHAPE),
    (dict(x=FAKE_X + 4), E_ARG),
    (dict(WT=FAKE_WT + 8), E_ARG),
])
def test_validation_rejects(kw, code):
    assert call(**kw) == code


def test_select_variant():
    lib = _lib.load()
    vs = _lib.variants()
    for d, io, units in [(64, 1, 2048), (64, 0, 256), (128, 0, 32), (16, 0, 16), (8, 0, 1)]:
        for n_lr in (4, 1):
            for reset in (0, 50):
                i = lib.srwm_select_variant(d, d, io, n_lr, reset, units)
                assert 0 <= i < len(vs)
                v = vs[i]
                assert (v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) == (d, d, "bf16" if io else "f32", n_lr)
                assert v["auto"] and (v["supports_reset"] or reset == 0)
    # many units: the fewest waves per unit; few units: more waves per unit
    assert vs[lib.srwm_select_variant(64, 64, 1, 4, 0, 2048)]["waves"] == 1
    assert vs[lib.srwm_select_variant(64, 64, 0, 4, 0, 256)]["waves"] > 1
    # one-wave units from two waves per SIMD on; multi-wave units fill four
    assert [vs[lib.srwm_select_variant(64, 64, 0, 4, 0, u)]["waves"] for u in (256, 512, 1024, 2048, 4096)] == \
        [8, 8, 4, 1, 1]
    assert lib.srwm_select_variant(7, 7, 0, 4, 0, 4) == E_UNSUP
    assert lib.srwm_select_variant(64, 64, 3, 4, 0, 4) == E_ARG
    assert lib.srwm_select_variant(64, 64, 0, 2, 0, 4) == E_ARG
    assert lib.srwm_select_variant(0, 64, 0, 4, 0, 4) == E_SHAPE


def test_variant_must_match_shape():
    vs = _lib.variants()
    v64 = next(v for v in vs if v["d_in"] == 64 and v["io_dtype"] == "f32")
    assert call(d_in=16, d_out=16, variant=v64["index"]) == E_ARG


def call_ex(**kw):
    base = dict(x=FAKE_X, W0=FAKE_W0, y=FAKE_Y, W_T=FAKE_WT, B=2, T=3, H=2, d_in=16, d_out=16,
                m=None, io_dtype=0, apply_input_softmax=0, n_lr=4, w0_per_sequence=0,
                reset_interval=0, variant=-1, stream=None)
    base.update(kw)
    if base["m"] is None:
        base["m"] = base["d_out"] + 2 * base["d_in"] + base["n_lr"]
    return _lib.load().srwm_forward_ex(ctypes.byref(_lib.ForwardArgs(**base)))


@pytest.mark.parametrize("kw,code", [
    (dict(t_stride=2), E_SHAPE),                    # sequences closer than T steps
    (dict(t_stride=-1), E_SHAPE),
    (dict(t_stride=1000, y=FAKE_X + 65536), E_ALIAS),  # y inside x's strided span
    (dict(n_lr=2), E_ARG),
    (dict(n_lr=1, m=52), E_SHAPE),
    (dict(n_lr=4, m=49), E_SHAPE),
    (dict(w0_per_sequence=2), E_ARG),
    (dict(reset_interval=-1), E_ARG),
    (dict(reset_interval=2 ** 40), E_ARG),
    (dict(W0=None, w0_per_sequence=1), E_NULL),
    (dict(W_T=FAKE_W0 + 8192, w0_per_sequence=1), E_ALIAS),  # inside the [B,H,m,d] W0 only
    (dict(d_in=7, d_out=7, n_lr=1), E_UNSUP),
])
def test_forward_ex_validation(kw, code):
    assert call_ex(**kw) == code


def test_forward_ex_null_args():
    assert _lib.load().srwm_forward_ex(None) == E_NULL


def test_fused_variant_rejects_reset():
    vs = _lib.variants()
    fused = next(v for v in vs if v["schedule"] == "fused" and v["d_in"] == 64 and v["io_dtype"] == "f32"
                 and v["n_lr"] == 4)
    assert not fused["supports_reset"]
    assert call_ex(d_in=64, d_out=64, variant=fused["index"], reset_interval=5) == E_ARG


def test_empty_problems_are_noops_without_gpu():
    # B*H == 0: nothing to do, no HIP call is made.
    assert call(B=0, x=None, y=None, WT=None) == OK
    assert call(H=0, x=None, y=None, W0=None, WT=None) == OK
    # T == 0 with no state requested: nothing to write.
    assert call(T=0, x=None, y=None, WT=None) == OK


# ---------------------------------------------------------------------------
# Backward pass and the forward tape.
FAKE_TAPE, FAKE_GY, FAKE_DX, FAKE_DWI, FAKE_DW0 = 0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000


def test_tape_row_and_backward_support():
    lib = _lib.load()
    for d_in, d_out, n_lr in [(8, 8, 4), (16, 16, 1), (64, 64, 4), (64, 64, 1), (3, 5, 1)]:
        m = d_out + 2 * d_in + n_lr
        assert lib.srwm_tape_row(d_in, d_out, n_lr) == (m + 3) // 4 * 4 + 3 * d_in + 4
    assert lib.srwm_tape_row(0, 8, 4) == E_SHAPE
    assert lib.srwm_tape_row(8, 8, 2) == E_SHAPE
    for d in (8, 16, 64):
        for io in (0, 1):
            for n_lr in (4, 1):
                assert lib.srwm_backward_supported(d, d, io, n_lr) == 1
    assert lib.srwm_backward_supported(128, 128, 0, 4) == 1
    assert lib.srwm_backward_supported(32, 32, 0, 4) == 0
    assert lib.srwm_backward_supported(64, 64, 2, 4) == 0
    # every shape with a backward kernel has forward variants that write the tape
    vs = _lib.variants()
    tape = {(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) for v in vs if v["writes_tape"]}
    for d in (8, 16, 64, 128):
        for io in ("f32", "bf16"):
            for n_lr in (4, 1):
                assert (d, d, io, n_lr) in tape
    # ... and, for the reset ablation, variants that write the tape and the windows' end states
    # (d = 128: no backward with resets)
    tape_reset = {(v["d_in"], v["d_out"], v["io_dtype"], v["n_lr"]) for v in vs
                  if v["writes_tape"] and v["supports_reset"]}
    assert tape_reset == {k for k in tape if k[0] != 128}


FAKE_WS = 0xB0000000


def test_forward_tape_validation():
    # with resets the tape needs the windows' end states (T = 3, R = 1: two resets)
    assert call_ex(tape=FAKE_TAPE, reset_interval=1) == E_NULL
    assert call_ex(tape=FAKE_TAPE, reset_interval=1, window_states=FAKE_WS + 4) == E_ARG
    assert call_ex(tape=FAKE_TAPE, reset_interval=1, window_states=FAKE_Y) == E_ALIAS
    assert call_ex(tape=FAKE_TAPE, reset_interval=1, window_states=FAKE_TAPE + 64) == E_ALIAS
    assert call_ex(tape=FAKE_TAPE + 4) == E_ARG                     # misaligned
    assert call_ex(tape=FAKE_X + 16) == E_ALIAS                     # overlaps x
    assert call_ex(tape=FAKE_TAPE, d_in=32, d_out=32) == E_UNSUP    # no tape variant at d=32
    vs = _lib.variants()
    plain = next(v for v in vs if v["d_in"] == 16 and v["io_dtype"] == "f32" and v["n_lr"] == 4
                 and not v["writes_tape"])
    taped = next(v for v in vs if v["d_in"] == 16 and v["io_dtype"] == "f32" and v["n_lr"] == 4
                 and v["writes_tape"])
    assert call_ex(tape=FAKE_TAPE, variant=plain["index"]) == E_ARG
    assert call_ex(variant=taped["index"]) == E_ARG


def call_bwd(**kw):
    base = dict(x=FAKE_X, W_T=FAKE_WT, tape=FAKE_TAPE, gy=FAKE_GY, gW_T=None, dx=FAKE_DX,
                dW_init=FAKE_DWI, dW0=FAKE_DW0, B=2, T=3, H=2, d_in=16, d_out=16, m=None,
                io_dtype=0, apply_input_softmax=0, n_lr=4, stream=None)
    base.update(kw)
    if base["m"] is None:
        base["m"] = base["d_out"] + 2 * base["d_in"] + base["n_lr"]
    return _lib.load().srwm_backward(ctypes.byref(_lib.BackwardArgs(**base)))


@pytest.mark.parametrize("kw,code", [
    (dict(n_lr=2), E_ARG),
    (dict(m=51), E_SHAPE),
    (dict(B=-1), E_SHAPE),
    (dict(d_in=0), E_SHAPE),
    (dict(io_dtype=2), E_ARG),
    (dict(apply_input_softmax=3), E_ARG),
    (dict(d_in=32, d_out=32), E_UNSUP),
    (dict(d_in=128, d_out=128, reset_interval=1), E_UNSUP),      # the wide kernel has no resets
    (dict(W_T=None), E_NULL),
    (dict(dW_init=None), E_NULL),
    (dict(tape=None), E_NULL),
    (dict(gy=None), E_NULL),
    (dict(dx=None), E_NULL),
    (dict(dx=FAKE_DX + 8), E_ARG),
    (dict(dx=FAKE_GY), E_ALIAS),
    (dict(dW0=FAKE_DWI + 16), E_ALIAS),
    (dict(gW_T=FAKE_DWI), E_ALIAS),
    (dict(dW_init=FAKE_TAPE + 64), E_ALIAS),
    (dict(reset_interval=-1), E_ARG),
    (dict(reset_interval=2 ** 40), E_ARG),
    (dict(reset_interval=1), E_NULL),                            # T = 3 > R: window states needed
    (dict(reset_interval=1, window_states=FAKE_WS + 8), E_ARG),
    (dict(reset_interval=1, window_states=FAKE_DWI), E_ALIAS),
])
def test_backward_validation(kw, code):
    assert call_bwd(**kw) == code


def call_bwd_noalloc(**kw):
    base = dict(x=FAKE_X, W_T=FAKE_WT, tape=FAKE_TAPE, gy=FAKE_GY, gW_T=None, dx=FAKE_DX,
                dW_init=None, dW0=FAKE_DW0, B=2, T=3, H=2, d_in=16, d_out=16, m=None,
                io_dtype=0, apply_input_softmax=0, n_lr=4, stream=None)
    base.update(kw)
    if base["m"] is None:
        base["m"] = base["d_out"] + 2 * base["d_in"] + base["n_lr"]
    return _lib.load().srwm_backward_noalloc(ctypes.byref(_lib.BackwardArgs(**base)))


@pytest.mark.parametrize("kw,code", [
    (dict(dW_init=FAKE_DWI), E_ARG),          # the per-unit gradients live in the library's scratch
    (dict(dW0=None), E_NULL),                 # the one gradient this entry point returns
    (dict(dx=None), E_NULL),
    (dict(m=51), E_SHAPE),
    (dict(d_in=32, d_out=32), E_UNSUP),
    (dict(dx=FAKE_GY), E_ALIAS),
    (dict(dW0=FAKE_TAPE + 16), E_ALIAS),
    (dict(dW0=FAKE_DW0 + 4), E_ARG),
    # one sequence's per-unit gradients (H*m*d_in floats) larger than the 32 MiB scratch
    (dict(H=200, d_in=128, d_out=128), E_SCRATCH),
    (dict(H=0, x=None, W_T=None, tape=None, gy=None, dx=None, dW0=None), OK),
])
def test_backward_noalloc_validation(kw, code):
    assert call_bwd_noalloc(**kw) == code


def test_backward_noalloc_scratch_size():
    assert _lib.load().srwm_backward_noalloc_scratch_bytes() == 32 << 20
    # the limit is one sequence's H*m*d_in floats: 168 heads of d = 128 fit, 169 do not
    assert 168 * 388 * 128 * 4 <= 32 << 20 < 169 * 388 * 128 * 4
    assert call_bwd_noalloc(H=169, d_in=128, d_out=128) == E_SCRATCH


def test_backward_null_and_empty():
    lib = _lib.load()
    assert lib.srwm_backward(None) == E_NULL
    assert call_bwd(B=0, x=None, W_T=None, tape=None, gy=None, dx=None, dW_init=None, dW0=None) == OK
    assert call_bwd(H=0, x=None, W_T=None, tape=None, gy=None, dx=None, dW_init=None, dW0=None) == OK


# ---------------------------------------------------------------------------
# DeltaNet / SR-DeltaNet entry points.
FAKE_Z = 0xA0000000


def call_dn(**kw):
    base = dict(x=FAKE_X, W_slow=FAKE_W0, F0=None, z=FAKE_Z, y=FAKE_Y, F_T=None, B=2, T=3, H=2, d_in=16,
                d_key=16, d_v=16, stream=None)
    base.update(kw)
    return _lib.load().srwm_deltanet_forward(ctypes.byref(_lib.DeltanetArgs(**base)))


def call_sdn(**kw):
    base = dict(x=FAKE_X, W0=FAKE_W0, F0=None, z=FAKE_Z, y=FAKE_Y, W_T=None, F_T=None, B=2, T=3, H=2, d_in=16,
                d_key=16, d_v=16, n_lr=4, apply_input_softmax=0, stream=None)
    base.update(kw)
    return _lib.load().srwm_srdeltanet_forward(ctypes.byref(_lib.SrdeltanetArgs(**base)))


def test_fwp_supported():
    lib = _lib.load()
    for d in (8, 16, 64):
        assert lib.srwm_fwp_supported(d, d) == 1
        P = 3 * d + 1
        for n_lr in (4, 1):
            assert lib.srwm_supported(d, P, 0, n_lr) == 1, (d, P, n_lr)
    assert lib.srwm_fwp_supported(7, 7) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(d_key=7, d_v=7), E_UNSUP),
    (dict(H=1, d_in=3), E_SHAPE),            # H*d_in not a multiple of 4
    (dict(B=-1), E_SHAPE),
    (dict(d_v=0), E_SHAPE),
    (dict(x=None), E_NULL),
    (dict(W_slow=None), E_NULL),
    (dict(z=None), E_NULL),
    (dict(y=None), E_NULL),
    (dict(y=FAKE_Y + 4), E_ARG),
    (dict(z=FAKE_X + 16), E_ALIAS),
    (dict(y=FAKE_Z + 64), E_ALIAS),
    (dict(F_T=FAKE_Y), E_ALIAS),
])
def test_deltanet_validation(kw, code):
    assert call_dn(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(n_lr=2), E_ARG),
    (dict(d_in=8, d_key=16, d_v=16), E_UNSUP),   # no SRWM kernel for d_out = 49 with d_in = 8
    (dict(d_key=7, d_v=7), E_UNSUP),
    (dict(y=FAKE_Y + 4), E_ARG),
    (dict(y=FAKE_Z + 64), E_ALIAS),
    (dict(F_T=FAKE_W0 + 16), E_ALIAS),
    # the SRWM half writes z and W_T before the fast matrix reads F0
    (dict(F0=FAKE_Z + 16), E_ALIAS),
    (dict(F0=FAKE_WT, W_T=FAKE_WT), E_ALIAS),
    (dict(F0=FAKE_WT + 64, W_T=FAKE_WT, F_T=FAKE_Y + 65536), E_ALIAS),
    (dict(y=None), E_NULL),
    (dict(chunk_steps=-1), E_ARG),
])
def test_srdeltanet_validation(kw, code):
    assert call_sdn(**kw) == code


def test_fwp_empty_problems_are_noops():
    lib = _lib.load()
    assert lib.srwm_deltanet_forward(None) == E_NULL
    assert lib.srwm_srdeltanet_forward(None) == E_NULL
    assert call_dn(B=0, x=None, z=None, y=None) == OK
    assert call_sdn(H=0, x=None, z=None, y=None, W0=None) == OK


def test_srdeltanet_chunk_steps():
    lib = _lib.load()
    # 256 units of an 8-wave projection leave room: about T/8 in 32-step pieces
    assert lib.srwm_srdeltanet_chunk_steps(128, 4096, 2, 64, 64, 64, 4) == 512
    assert lib.srwm_srdeltanet_chunk_steps(128, 1000, 2, 64, 64, 64, 1) == 256   # at least 256
    assert lib.srwm_srdeltanet_chunk_steps(128, 3000, 2, 64, 64, 64, 4) == 384   # ceil(375 / 32) * 32
    # a projection that fills the chip: no chunks (T)
    assert lib.srwm_srdeltanet_chunk_steps(1024, 4096, 16, 64, 64, 64, 4) == 4096
    assert lib.srwm_srdeltanet_chunk_steps(2, 3, 2, 16, 16, 16, 2) == E_ARG
    assert lib.srwm_srdeltanet_chunk_steps(2, 3, 2, 16, 7, 7, 4) == E_UNSUP
    assert lib.srwm_srdeltanet_chunk_steps(-1, 3, 2, 16, 16, 16, 4) == E_SHAPE


def test_struct_layouts_match_the_header(tmp_path):
    # The ctypes mirrors of the argument structs against the C compiler's
    # layout of include/srwm.h: every field's offset, and the size.
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    structs = {"srwm_forward_args_t": _lib.ForwardArgs, "srwm_backward_args_t": _lib.BackwardArgs,
               "srwm_deltanet_args_t": _lib.DeltanetArgs, "srwm_srdeltanet_args_t": _lib.SrdeltanetArgs,
               "srwm_fast_args_t": _lib.FastArgs, "srwm_variant_info_t": _lib.VariantInfo,
               "srwm_kernel_resources_t": _lib.KernelResources}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "srwm.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in cls._fields_:
            lines.append(f'printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    inc = Path(__file__).resolve().parents[1] / "include"
    subprocess.check_call(["gcc", "-std=c11", "-I", str(inc), str(src), "-o", str(tmp_path / "layout")])
    got = dict(line.rsplit(" ", 1) for line in
               subprocess.check_output([str(tmp_path / "layout")], text=True).splitlines())
    for cname, cls in structs.items():
        assert int(got[f"{cname} size"]) == ctypes.sizeof(cls), cname
        for f in cls._fields_:
            assert int(got[f"{cname} {f[0]}"]) == getattr(cls, f[0]).offset, (cname, f[0])


def call_fast(**kw):
    base = dict(z=FAKE_Z, F0=None, y=FAKE_Y, F_T=None, B=2, T=3, H=2, d_key=16, d_v=16, stream=None)
    base.update(kw)
    return _lib.load().srwm_fast_forward(ctypes.byref(_lib.FastArgs(**base)))


@pytest.mark.parametrize("kw,code", [
    (dict(d_key=7, d_v=7), E_UNSUP),
    (dict(T=-1), E_SHAPE),
    (dict(z=None), E_NULL),
    (dict(y=None), E_NULL),
    (dict(F_T=FAKE_Y + 4), E_ARG),
    (dict(y=FAKE_Z + 32), E_ALIAS),
    (dict(F_T=FAKE_Y + 64), E_ALIAS),
    (dict(t_stride=2), E_SHAPE),
    (dict(t_stride=1000, y=FAKE_Z + 65536), E_ALIAS),
])
def test_fast_forward_validation(kw, code):
    assert call_fast(**kw) == code


def test_deltanet_project_ignores_fast_buffers():
    # the projection alone needs no y; its checks still reject bad shapes
    assert call_dn(B=0, x=None, z=None, y=None) == OK
    lib = _lib.load()
    a = _lib.DeltanetArgs(x=FAKE_X, W_slow=FAKE_W0, F0=None, z=FAKE_Z, y=None, F_T=None, B=2, T=3, H=1,
                          d_in=3, d_key=16, d_v=16, stream=None)
    assert lib.srwm_deltanet_project(ctypes.byref(a)) == E_SHAPE
    a = _lib.DeltanetArgs(x=FAKE_X, W_slow=FAKE_W0, F0=None, z=FAKE_X + 16, y=None, F_T=None, B=2, T=3, H=2,
                          d_in=16, d_key=16, d_v=16, stream=None)
    assert lib.srwm_deltanet_project(ctypes.byref(a)) == E_ALIAS


def test_size_limits():
    # the kernels index units and steps with 32-bit grid coordinates: B*H and T
    # must fit, else SRWM_ERR_SHAPE before any device call
    assert call(B=2 ** 31, H=1, T=1) == E_SHAPE
    assert call(B=1, H=1, T=2 ** 31) == E_SHAPE
    assert call_ex(B=2 ** 16, H=2 ** 16, T=1) == E_SHAPE
    # a chunk of x is addressed with 32-bit lane offsets: a step's row of x
    # (H*d_in elements) may span at most 64 MiB
    assert call(B=1, H=2 ** 20 + 1, T=1) == E_SHAPE  # fp32, d_in = 16
    assert call(B=1, H=2 ** 21 + 1, T=1, io=1) == E_SHAPE  # bf16
    assert call_bwd(B=2 ** 31, H=1, T=1) == E_SHAPE
    assert call_bwd(T=2 ** 31, B=1, H=1) == E_SHAPE
    assert call_dn(B=2 ** 31, H=1, T=1) == E_SHAPE
    assert call_fast(B=1, H=1, T=2 ** 31) == E_SHAPE
    assert _lib.load().srwm_tape_row(2 ** 40, 1, 4) > 0  # large but well-formed row lengths are computed


def test_valu_probe_validation():
    lib = _lib.load()
    assert lib.srwm_valu_probe(None, 4, 1, None) == E_NULL
    assert lib.srwm_valu_probe(FAKE_Y, 0, 1, None) == E_SHAPE
    assert lib.srwm_valu_probe(FAKE_Y, 4, 0, None) == E_SHAPE
    assert lib.srwm_valu_probe(FAKE_Y + 4, 4, 1, None) == E_ARG
    assert lib.srwm_valu_probe_flop(2, 3) == 2 * 256 * 3 * 16 * 8 * 2


def test_lds_probe_validation():
    lib = _lib.load()
    assert lib.srwm_lds_probe(None, 4, 1, None) == E_NULL
    assert lib.srwm_lds_probe(FAKE_Y, 0, 1, None) == E_SHAPE
    assert lib.srwm_lds_probe(FAKE_Y, 4, 0, None) == E_SHAPE
    assert lib.srwm_lds_probe(FAKE_Y + 4, 4, 1, None) == E_ARG
    # 16 reads of 16 bytes per lane and iteration
    assert lib.srwm_lds_probe_bytes(2, 3) == 2 * 256 * 3 * 16 * 16


# ---------------------------------------------------------------------------
# Kernel resource queries: validation before any HIP call.
def test_resource_query_validation():
    lib = _lib.load()
    r = _lib.KernelResources()
    n = lib.srwm_variant_count()
    assert lib.srwm_variant_resources(-1, ctypes.byref(r)) == E_ARG
    assert lib.srwm_variant_resources(n, ctypes.byref(r)) == E_ARG
    assert lib.srwm_variant_resources(0, None) == E_NULL
    assert lib.srwm_backward_resources(64, 64, 2, 0, 1, ctypes.byref(r)) == E_ARG
    assert lib.srwm_backward_resources(64, 64, 4, 0, -1, ctypes.byref(r)) == E_SHAPE
    assert lib.srwm_backward_resources(64, 64, 4, 0, 1, None) == E_NULL
    assert lib.srwm_backward_resources(32, 32, 4, 0, 1, ctypes.byref(r)) == E_UNSUP
    assert lib.srwm_backward_resources(128, 128, 4, 1, 1, ctypes.byref(r)) == E_UNSUP  # no wide reset kernel
