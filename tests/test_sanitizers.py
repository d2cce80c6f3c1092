"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

1. The float64 / float32 oracle (oracle/srwm_oracle.c), built with gcc and
   the sanitizers, run over the shapes its pins use (tests/sanitize/
   oracle_driver.c): the pointer arithmetic over [B][T][H][d] and the thread
   pool must stay in bounds, leak nothing and do nothing undefined.
2. libsrwm's host code (argument validation, size-overflow checks, aliasing,
   variant choice), built with the sanitizers on the host side only, driven
   through every error path that is decided before a HIP call
   (tests/sanitize/abi_driver.c).  Nothing reaches a GPU.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SAN = ROOT / "tests" / "sanitize"
CSRC = ROOT / "self_referential_weight_amd" / "csrc"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    cflags = ["-O1", "-g", "-ffp-contract=off", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    src = ROOT / "oracle" / "srwm_oracle.c"
    objs = []
    for tag, extra in (("f64", []), ("f32", ["-DORACLE_FLOAT"])):
        o = tmp_path / f"oracle_{tag}.o"
        run(["gcc", *cflags, *extra, "-c", str(src), "-o", str(o)])
        objs.append(str(o))
    drv = tmp_path / "oracle_driver"
    run(["gcc", *cflags, str(SAN / "oracle_driver.c"), *objs, "-lm", "-lpthread", "-o", str(drv)])
    r = run([str(drv)], env=ENV, timeout=300)
    assert "oracle_driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


def _rocm_tool(name):
    for cand in (shutil.which(name), f"/opt/rocm/bin/{name}", f"/opt/rocm/llvm/bin/{name}"):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc, clang, clangxx = _rocm_tool("hipcc"), _rocm_tool("clang"), _rocm_tool("clang++")
    if not (hipcc and clang and clangxx):
        pytest.skip("ROCm toolchain not available")
    # sanitizers on the host side of each object only (the device code is
    # compiled as usual): every -fsanitize= sits right after -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-I", str(ROOT / "include"),
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san]
    srcs = sorted(CSRC.glob("*.hip"))
    objs = [tmp_path / (s.stem + ".o") for s in srcs]
    procs = [subprocess.Popen([hipcc, *flags, "-c", str(s), "-o", str(o)], stdout=subprocess.PIPE,
                              stderr=subprocess.PIPE, text=True) for s, o in zip(srcs, objs)]
    for p, s in zip(procs, srcs):
        out, err = p.communicate(timeout=900)
        assert p.returncode == 0, f"{s.name}\n{err[-3000:]}"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    drv_o = tmp_path / "abi_driver.o"
    run([clang, "-O1", "-g", *san, "-I", str(ROOT / "include"), "-c", str(SAN / "abi_driver.c"), "-o", str(drv_o)])
    exe = tmp_path / "abi_driver"
    run([clangxx, *san, "-o", str(exe), str(drv_o), *map(str, objs), "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib"])
    r = run([str(exe)], env=ENV, timeout=300)
    assert "abi_driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
