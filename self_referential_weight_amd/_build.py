"""Build libsrwm.so (gfx950) in-tree with hipcc: each source compiles to an
object in parallel, then one link."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SRCS = [PKG / "csrc" / f for f in ("srwm_fwd_d64.hip", "srwm_fwd_tape.hip", "srwm_fwd_misc.hip", "srwm_fwd_small.hip",
                                    "srwm_bwd.hip", "srwm_fwd.hip", "srwm_fwp.hip", "srwm_calib.hip")]
LIB = PKG / "libsrwm.so"

HIPCC_FLAGS = [
    "-O3",
    "--offload-arch=gfx950",
    "-std=c++17",
    "-fPIC",
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
    cc = hipcc()
    srcs = SRCS
    with tempfile.TemporaryDirectory(prefix="srwm_build_") as tmpdir:
        objs = [Path(tmpdir) / (s.stem + ".o") for s in srcs]
        cmds = [[cc, *HIPCC_FLAGS, "-I", str(ROOT / "include"), "-c", str(s), "-o", str(o)]
                for s, o in zip(srcs, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), cmds))
        for c, r in zip(cmds, results):
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(c)}\n{r.stdout}{r.stderr}")
        tmp = LIB.with_name(LIB.name + ".tmp")
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", str(tmp), *[str(o) for o in objs]]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
