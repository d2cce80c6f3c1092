"""Build libsrwm.so (gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRCS = [PKG / "csrc" / f for f in ("srwm_fwd.hip", "srwm_bwd.hip", "srwm_fwp.hip", "srwm_calib.hip")]
LIB = PKG / "libsrwm.so"

HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Packed FP32 (v_pk_fma_f32 and friends) stays off: every FMA is scalar.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsrwm)")


def build(verbose: bool = False) -> Path:
    """Compile the kernels and the C ABI into self_referential_weight_amd/libsrwm.so."""
    tmp = LIB.with_name(LIB.name + ".tmp")
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", str(ROOT / "include"), "-o", str(tmp), *[str(f) for f in SRCS]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
