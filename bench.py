"""Throughput of the SRWM forward recurrence on one MI355X.

One "step" is one srwm_forward call over a whole synthetic batch (every
(sequence, head) unit through all T time steps).  The default workload is the
RL-shaped one: B=128, H=16, d_in=d_out=64 (m=196), T=4096, bf16 x/y, fp32
state, softmax on x_t.  Inputs are seeded, generated on the host and resident
in HBM before timing starts.

Prints ONE JSON line with the headline metric (head-steps/s = B*H*T/s), the
roofline of the kernel (algorithmic FP32 FLOP per launch / average launch time
from HIP events on the launch stream, against the FP32 vector peak) and the
float64 CPU oracle timed on a bounded sample of the same workload.  After the
timed headline steps, the `configs` block times every SRWM workload the same
way (median and minimum launch time, head-steps/s, fraction of the FP32 peak)
beside the oracle on a bounded sample of each, and `calibration` holds the
chip's measured scalar FMA rate and LDS read bandwidth.

With --backward a step is one training pass instead: the forward pass that
records the tape, then the backward pass (dx and the batch-summed dW0 for a
seeded output cotangent); the roofline then describes the backward kernel and
the CPU baseline is the float64 gradient oracle.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--variant I] [--no-cpu] [--copy-calibration BYTES] [--backward]
                  [--no-configs] [--config-cpu-budget S]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "SRWM head-steps/sec (B·H·T/s) and % of FP32 VALU peak, 1×MI355X"
# MI355X FP32 vector peak: 256 CUs x 256 FLOP/clk/CU x 2.4 GHz.
PEAK_FP32_TFLOPS = 157.3
# The forward kernels' device code and the device helpers they include (the
# variant table and host code do not change the kernel's traffic).
KERNEL_SRCS = [ROOT / "self_referential_weight_amd" / "csrc" / f for f in ("srwm_fwd_kernels.h", "srwm_device.h")]
TRAFFIC_FILE = ROOT / "profiles" / "srwm_fwd_rl_d64_bf16_hbm_traffic.json"
# The backward kernel's device code and the device helpers it includes.
BWD_SRCS = [ROOT / "self_referential_weight_amd" / "csrc" / f for f in ("srwm_bwd_kernels.h", "srwm_device.h")]
BWD_TRAFFIC_FILE = ROOT / "profiles" / "srwm_bwd_rl_d64_bf16_hbm_traffic.json"
LDS_FILE = ROOT / "profiles" / "srwm_lds_rl_d64_bf16.json"
# LDS bandwidth the achieved figure is compared with: 128 bytes per clock per
# CU (the CDNA3 compute unit's figure, assumed) x 256 CUs x 2.4 GHz.
PEAK_LDS_TBPS = 128 * 256 * 2.4e9 / 1e12


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(srcs=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SRCS if srcs is None else srcs):
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, variant: int, path=TRAFFIC_FILE, srcs=None):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, if they were taken on the current kernel source; else None."""
    if not path.exists():
        return None
    try:
        rec = json.loads(path.read_text())
    except ValueError:
        return None
    if (rec.get("kernel_source_sha256_16") != kernel_source_hash(srcs)
            or rec.get("workload") != workload or rec.get("variant", -1) != variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def valu_calibration(dev, stream) -> dict:
    """The chip's measured scalar FP32 FMA rate (srwm_valu_probe: independent
    FMA chains over 8 waves per SIMD), outside the timed region."""
    import torch

    from self_referential_weight_amd import _lib

    lib = _lib.load()
    wgs, iters = 2048, 12000
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    handle = stream.cuda_stream
    rc = lib.srwm_valu_probe(out.data_ptr(), wgs, iters, handle)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        lib.srwm_valu_probe(out.data_ptr(), wgs, iters, handle)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    return {"fp32_scalar_fma_TFLOPs": lib.srwm_valu_probe_flop(wgs, iters) / (ms * 1e-3) / 1e12,
            "probe": f"{wgs} workgroups x 256 threads x {iters * 16} x 8 independent v_fma_f32 chains"}


def lds_calibration(dev, stream) -> dict:
    """The chip's measured LDS read bandwidth (srwm_lds_probe: conflict-free
    16-byte LDS reads by every lane, 8 workgroups of 4 waves per CU), outside
    the timed region."""
    import torch

    from self_referential_weight_amd import _lib

    lib = _lib.load()
    wgs, iters = 2048, 4096
    out = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    handle = stream.cuda_stream
    rc = lib.srwm_lds_probe(out.data_ptr(), wgs, iters, handle)
    if rc != 0:
        raise RuntimeError(_lib.strerror(rc))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        lib.srwm_lds_probe(out.data_ptr(), wgs, iters, handle)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    tbps = lib.srwm_lds_probe_bytes(wgs, iters) / (ms * 1e-3) / 1e12
    return {"lds_read_TBps": tbps, "bytes_per_clk_per_cu_at_2.4GHz": tbps * 1e12 / (256 * 2.4e9),
            "probe": f"{wgs} workgroups x 256 threads x {iters * 16} ds_read_b128, conflict-free"}


def measured_lds(which: str, workload: str, srcs, kernel_ms: float, peak_tbps=None):
    """LDS bytes per launch from the committed counter run, if taken on the
    current kernel source and workload, turned into a rate over kernel_ms and
    compared with the measured LDS read bandwidth (peak_tbps) when given, else
    with the assumed CDNA3 figure."""
    if not LDS_FILE.exists():
        return None
    try:
        rec = json.loads(LDS_FILE.read_text()).get(which, {})
    except ValueError:
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(srcs) or rec.get("workload") != workload:
        return None
    nbytes = rec["lds_load_bytes_per_launch"] + rec["lds_store_bytes_per_launch"]
    tbps = nbytes / (kernel_ms * 1e-3) / 1e12
    peak = peak_tbps if peak_tbps else PEAK_LDS_TBPS
    return {"bytes_per_launch": nbytes, "achieved": tbps, "unit": "TB/s", "peak": peak,
            "peak_kind": "measured (srwm_lds_probe)" if peak_tbps else "assumed (128 B/clk/CU)",
            "frac": tbps / peak}


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x_host, W0_host, budget_s: float):
    """Time the float64 oracle on the first n sequences (all heads, all T
    steps) of the workload, n sized so the run takes about budget_s."""
    import numpy as np

    from oracle import oracle

    cores = oracle.default_threads()
    # calibration: one sequence
    t0 = time.perf_counter()
    oracle.forward(np.ascontiguousarray(x_host[:1], dtype=np.float64), W0_host,
                   w.apply_input_softmax, return_state=False, nthreads=cores)
    t1 = time.perf_counter() - t0
    # one thread takes tau seconds per unit; n sequences spread n*H units over the cores
    tau = t1 * min(w.H, cores) / w.H
    n = max(1, min(w.B, int(budget_s * cores / (max(tau, 1e-9) * w.H))))
    xs = np.ascontiguousarray(x_host[:n], dtype=np.float64)
    # very small workloads: repeat the call until the wall time is measurable
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(xs, W0_host, w.apply_input_softmax, return_state=False, nthreads=cores)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min(0.5, budget_s) or reps >= 100000:
            break
    units = n * w.H
    rep_note = f", {reps} repetitions" if reps > 1 else ""
    return {
        "value": reps * units * w.T / dt,
        "unit": "head-steps/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"first {n} of {w.B} sequences x {w.H} heads ({units} units) x T={w.T} "
                   f"of {w.name}, float64, {dt:.1f} s wall{rep_note}"),
    }


def oracle_cores_note() -> dict:
    """How many host CPUs the oracle's thread pool uses and why."""
    from oracle import oracle

    try:
        aff = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = os.cpu_count() or 1
    return {"affinity_cpus": aff, "threads": oracle.default_threads(),
            "cap": "at most 16 threads (and OMP_NUM_THREADS): the host share one GPU is allotted"}


def time_launches(step, stream, steps: int, warmup: int) -> list:
    """Per-launch durations (ms) of `step` from HIP events on `stream`, one
    event between consecutive launches, after `warmup` untimed calls."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]


def median(v: list) -> float:
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def config_entry(w, per_launch: list, fma_rate, cpu) -> dict:
    """One workload's line of the `configs` block."""
    import self_referential_weight_amd as srwm

    med, mn = median(per_launch), min(per_launch)
    flop = w.flop_per_head_step * w.head_steps
    kernel = srwm.select_variant(w.d_in, w.d_out, w.io_dtype, w.units)
    ent = {
        "B": w.B, "H": w.H, "d_in": w.d_in, "d_out": w.d_out, "T": w.T, "io_dtype": w.io_dtype,
        "apply_input_softmax": w.apply_input_softmax, "return_state": w.return_state,
        "units": w.units, "launches": len(per_launch),
        "ms_median": med, "ms_min": mn, "ms_mean": sum(per_launch) / len(per_launch),
        "head_steps_per_s": w.head_steps / (med * 1e-3),
        "frac": flop / (med * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "executed_frac": 0.75 * flop / (med * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "kernel": f"srwm_fwd_kernel<{w.d_in},{w.d_out},{kernel['waves']},{kernel['lanes_per_row']},"
                  f"{kernel['waves_per_simd']},...> ({kernel['schedule']}, variant {kernel['index']})",
    }
    if fma_rate:
        ent["executed_frac_of_measured_fma_rate"] = 0.75 * flop / (med * 1e-3) / 1e12 / fma_rate
    if cpu is not None:
        ent["cpu_baseline"] = cpu
    return ent


def copy_calibration(nbytes: int, dev) -> None:
    """Three plain device-to-device copies of nbytes (scale reference for the
    HBM byte counters)."""
    import torch

    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    bcopy = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        bcopy.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: 3 copies of {nbytes} bytes done")


def cpu_baseline_backward(w, x_host, W0_host, gy_host, budget_s: float):
    """Time the float64 gradient oracle on the first n sequences, n sized from
    a calibration run on a prefix of one sequence so the run takes about budget_s."""
    import numpy as np
    import torch

    from oracle import backward as oracle_bwd

    cores = torch.get_num_threads()
    Tc = min(w.T, 64)
    t0 = time.perf_counter()
    oracle_bwd.grads(x_host[:1, :Tc], W0_host, w.apply_input_softmax, gy_host[:1, :Tc], n_lr=w.n_lr)
    per_step = (time.perf_counter() - t0) / Tc          # seconds per step of one sequence
    # autograd over a longer, batched run costs about twice the prefix's rate per step
    n = max(1, min(w.B, int(budget_s / (2.0 * per_step * w.T))))
    T = w.T
    if n == 1 and 2.0 * per_step * w.T > budget_s:
        T = max(1, int(budget_s / (2.0 * per_step)))
    t0 = time.perf_counter()
    oracle_bwd.grads(np.ascontiguousarray(x_host[:n, :T]), W0_host, w.apply_input_softmax,
                     np.ascontiguousarray(gy_host[:n, :T]), n_lr=w.n_lr)
    dt = time.perf_counter() - t0
    units = n * w.H
    return {
        "value": units * T / dt,
        "unit": "head-steps/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"forward+backward of the first {n} of {w.B} sequences x {w.H} heads ({units} units) "
                   f"x T={T} of {w.name}, float64 autograd, {dt:.1f} s wall"),
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--variant", type=int, default=-1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle wall time")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time the training step (taped forward + backward) instead of the forward")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the `configs` block (every SRWM workload timed after the headline)")
    ap.add_argument("--config-cpu-budget", type=float, default=3.0,
                    help="seconds of oracle wall time per workload in the `configs` block")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: libsrwm measures one GPU only (--gpus {args.gpus} requested); "
              "the (sequence, head) units shard across GPUs with no communication, "
              "so one GPU's share is what is measured", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: multi-rank launch is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import self_referential_weight_amd as srwm
    from self_referential_weight_amd.workloads import HEADLINE, WORKLOADS, gen_W0, gen_x

    name = args.workload or HEADLINE
    from self_referential_weight_amd.workloads import FWP_WORKLOADS
    if name in FWP_WORKLOADS:
        return bench_fwp(args, FWP_WORKLOADS[name])
    w = WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"[bench] generating {name}: B={w.B} H={w.H} d_in={w.d_in} d_out={w.d_out} T={w.T} "
        f"io={w.io_dtype} input_softmax={w.apply_input_softmax}")
    x_host = gen_x(w)
    W0_host = gen_W0(w)
    x = torch.from_numpy(x_host).to(dev)
    if w.io_dtype == "bf16":
        x = x.to(torch.bfloat16)
    W0 = torch.from_numpy(W0_host).to(dev)
    y = torch.empty((w.B, w.T, w.H, w.d_out), dtype=x.dtype, device=dev)
    W_T = torch.empty((w.B, w.H, w.m, w.d_in), dtype=torch.float32, device=dev) if w.return_state else None
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration:
        copy_calibration(int(args.copy_calibration), dev)

    if args.backward:
        return bench_backward(args, w, name, x, x_host, W0, W0_host, dev)

    def step():
        srwm.forward(x, W0, apply_input_softmax=w.apply_input_softmax, return_state=w.return_state,
                     variant=args.variant, y=y, W_T=W_T, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")

    # one event between consecutive launches: per-launch durations, same stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    gpu_ms = evs[0].elapsed_time(evs[-1]) / args.steps  # one kernel launch per step
    med_ms = median(per_launch)
    ms_per_step = wall * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step wall, {gpu_ms:.3f} ms/launch (HIP events)")

    head_steps = w.B * w.H * w.T
    flop = w.flop_per_head_step * head_steps
    achieved = flop / (gpu_ms * 1e-3) / 1e12
    io_bytes = head_steps * (w.d_in + w.d_out) * (2 if w.io_dtype == "bf16" else 4)
    traffic = measured_traffic(name, args.variant)
    kernel = (srwm.variants()[args.variant] if args.variant >= 0
              else srwm.select_variant(w.d_in, w.d_out, w.io_dtype, w.units))

    # Chip calibrations, outside the timed region: the scalar FP32 FMA rate and
    # the LDS read bandwidth.
    cal = valu_calibration(dev, stream)
    lds_cal = lds_calibration(dev, stream)
    rec = {
        "metric": METRIC,
        "value": head_steps / (ms_per_step * 1e-3),
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal x, W0 ~ N(0, 1/d_in); no dataset)",
        "config": {"workload": name, "B": w.B, "H": w.H, "d_in": w.d_in, "d_out": w.d_out,
                   "T": w.T, "io_dtype": w.io_dtype, "apply_input_softmax": w.apply_input_softmax,
                   "return_state": w.return_state, "variant": args.variant},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS, "traffic": traffic},
        "kernel": dict({k: kernel[k] for k in ("index", "waves", "lanes_per_row", "waves_per_simd", "schedule")},
                       resources=srwm.kernel_resources(kernel["index"])),
        "lds": (measured_lds("forward", name, None, gpu_ms, lds_cal["lds_read_TBps"])
                if args.variant < 0 else None),
        "kernel_ms": gpu_ms,
        "kernel_ms_median": med_ms,
        "kernel_ms_min": min(per_launch),
        "io_stream_GBps": io_bytes / (gpu_ms * 1e-3) / 1e9,
    }
    # Against the measured scalar FP32 rate: the kernel executes 6 m d_in FLOP
    # per head-step (the two reads fused into one) of the algorithmic 8 m d_in.
    executed = achieved * 6.0 / 8.0
    cal.update({"executed_TFLOPs": executed, "executed_frac": executed / cal["fp32_scalar_fma_TFLOPs"]})
    rec["calibration"] = dict(cal, lds=lds_cal)
    log(f"[bench] measured scalar FP32 FMA rate {cal['fp32_scalar_fma_TFLOPs']:.1f} TFLOP/s; "
        f"kernel executes {executed:.1f} TFLOP/s ({100 * cal['executed_frac']:.1f}%); "
        f"LDS read {lds_cal['lds_read_TBps']:.1f} TB/s")
    if not args.no_cpu:
        log("[bench] timing the float64 CPU oracle on a bounded sample")
        rec["cpu_baseline"] = dict(cpu_baseline(w, x_host, W0_host, args.cpu_budget), **oracle_cores_note())
    if not args.no_configs and args.variant < 0:
        rec["configs"] = all_configs(args, name, w, per_launch, rec.get("cpu_baseline"), dev, stream,
                                     cal["fp32_scalar_fma_TFLOPs"])
    print(json.dumps(rec), flush=True)
    return 0


def all_configs(args, headline, hw, headline_launches, headline_cpu, dev, stream, fma_rate) -> dict:
    """Every SRWM workload, timed like the headline (HIP events around each
    launch of the automatically chosen kernel on `stream`, after warm-up),
    with the float64 oracle timed on a bounded sample of each.  The headline
    workload reuses the timed launches above."""
    import torch

    import self_referential_weight_amd as srwm
    from self_referential_weight_amd.workloads import WORKLOADS, gen_W0, gen_x

    out = {}
    for name, w in WORKLOADS.items():
        if name == headline:
            out[name] = config_entry(hw, headline_launches, fma_rate, headline_cpu)
            continue
        x_host, W0_host = gen_x(w), gen_W0(w)
        x = torch.from_numpy(x_host).to(dev)
        if w.io_dtype == "bf16":
            x = x.to(torch.bfloat16)
        W0 = torch.from_numpy(W0_host).to(dev)
        y = torch.empty((w.B, w.T, w.H, w.d_out), dtype=x.dtype, device=dev)
        W_T = torch.empty((w.B, w.H, w.m, w.d_in), dtype=torch.float32, device=dev) if w.return_state else None

        def step():
            srwm.forward(x, W0, apply_input_softmax=w.apply_input_softmax, return_state=w.return_state,
                         y=y, W_T=W_T, stream=stream)
        launches = time_launches(step, stream, max(args.steps, 20), max(args.warmup, 3))
        log(f"[bench] {name}: median {median(launches):.4f} ms, min {min(launches):.4f} ms "
            f"over {len(launches)} launches")
        cpu = None
        if not args.no_cpu:
            cpu = dict(cpu_baseline(w, x_host, W0_host, args.config_cpu_budget), **oracle_cores_note())
        out[name] = config_entry(w, launches, fma_rate, cpu)
        del x, W0, y, W_T
    return out


def bench_backward(args, w, name, x, x_host, W0, W0_host, dev) -> int:
    import torch

    import self_referential_weight_amd as srwm
    from self_referential_weight_amd.workloads import gen_gy

    gy_host = gen_gy(w)
    gy = torch.from_numpy(gy_host).to(dev)
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd_ms, bwd_ms = [], []

    def step(timed: bool):
        if timed:
            ev[0].record(stream)
        y, W_T, tape = srwm.forward(x, W0, apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr,
                                    save_tape=True, stream=stream)
        if timed:
            ev[1].record(stream)
        srwm.backward(x, W_T, tape, gy, None, apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr,
                      shared_W0=True, stream=stream)
        if timed:
            ev[2].record(stream)
            torch.cuda.synchronize()
            fwd_ms.append(ev[0].elapsed_time(ev[1]))
            bwd_ms.append(ev[1].elapsed_time(ev[2]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} training steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    f_ms = sum(fwd_ms) / len(fwd_ms)
    b_ms = sum(bwd_ms) / len(bwd_ms)
    log(f"[bench] {args.steps} training steps: {ms_per_step:.3f} ms/step wall; "
        f"forward {f_ms:.3f} ms, backward {b_ms:.3f} ms (HIP events)")
    head_steps = w.B * w.H * w.T
    # Algorithmic work of the backward per head-step, counted like the
    # forward's 8 m d_in: each of the three matrix-vector products (W u, W qh,
    # W kh) has two adjoint products (the vector's and the matrix's, 4 m d_in
    # FLOP), the rank-one update two more (Wh kh and Wh^T a, 4 m d_in): 16 m d_in.
    flop_bwd = 16 * w.m * w.d_in * head_steps
    achieved = flop_bwd / (b_ms * 1e-3) / 1e12
    lds_cal = lds_calibration(dev, stream)
    rec = {
        "metric": "SRWM training head-steps/sec (taped forward + backward), 1×MI355X",
        "value": head_steps / (ms_per_step * 1e-3),
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal x, W0 ~ N(0, 1/d_in), normal output cotangent; no dataset)",
        "config": {"workload": name + "+backward", "B": w.B, "H": w.H, "d_in": w.d_in, "d_out": w.d_out,
                   "T": w.T, "io_dtype": w.io_dtype, "apply_input_softmax": w.apply_input_softmax},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS,
                     "traffic": measured_traffic(name + "+backward", -1, BWD_TRAFFIC_FILE, BWD_SRCS)},
        "lds": measured_lds("backward", name + "+backward", BWD_SRCS, b_ms, lds_cal["lds_read_TBps"]),
        "calibration": {"lds": lds_cal},
        "forward_ms": f_ms,
        "backward_ms": b_ms,
        "backward_kernel_resources": srwm.backward_resources(w.d_in, w.d_out, w.n_lr, False, w.units),
    }
    if not args.no_cpu:
        log("[bench] timing the float64 gradient oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline_backward(w, x_host, W0_host, gy_host, args.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


def bench_fwp(args, w) -> int:
    """DeltaNet / SR-DeltaNet: a step is the projection of every (b, t) (the
    MFMA GEMM, or the SRWM kernel for SR-DeltaNet) and the fast-matrix
    recurrence.  DeltaNet runs them one after the other, each launch bracketed
    by HIP events; SR-DeltaNet runs the library's overlapped schedule (time
    chunks, the two halves on two streams)."""
    import numpy as np
    import torch

    import self_referential_weight_amd as srwm
    from self_referential_weight_amd.workloads import gen_W0, gen_W_slow, gen_x

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(int(args.copy_calibration), dev)
    log(f"[bench] generating {w.name}: {w.kind} B={w.B} H={w.H} d_in={w.d_in} d_key={w.d_key} d_v={w.d_v} T={w.T}")
    x_host = gen_x(w)
    x = torch.from_numpy(x_host).to(dev)
    P = w.P
    z = torch.empty((w.B, w.T, w.H, P), dtype=torch.float32, device=dev)
    y = torch.empty((w.B, w.T, w.H, w.d_v), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if w.kind == "deltanet":
        Wp_host = gen_W_slow(w)
        Wp = torch.from_numpy(Wp_host).to(dev)

        def project():
            srwm.deltanet_project(x, Wp, w.d_key, w.d_v, z=z, stream=stream)
        proj_name = "srwm_proj_gemm_kernel"
        proj_flop = 2 * P * w.H * w.d_in * w.head_steps
        proj_bound, proj_unit = "mfma", "TFLOP/s"
    else:
        Wp_host = gen_W0(w)
        Wp = torch.from_numpy(Wp_host).to(dev)

        def project():
            srwm.forward(x, Wp, apply_input_softmax=w.apply_input_softmax, n_lr=w.n_lr, y=z, stream=stream)
        proj_name = "srwm_fwd_kernel (SRWM, d_out = P)"
        proj_flop = 8 * w.m * w.d_in * w.head_steps
        proj_bound, proj_unit = "alu", "TFLOP/s"

    fast_flop = 6 * w.d_v * w.d_key * w.head_steps
    if w.kind == "deltanet":
        def fast():
            srwm.fast_forward(z, w.d_key, w.d_v, y=y, stream=stream)

        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        t_proj, t_fast = [], []
        for _ in range(args.warmup):
            project()
            fast()
        torch.cuda.synchronize()
        log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
        t0 = time.perf_counter()
        for _ in range(args.steps):
            ev[0].record(stream)
            project()
            ev[1].record(stream)
            fast()
            ev[2].record(stream)
            torch.cuda.synchronize()
            t_proj.append(ev[0].elapsed_time(ev[1]))
            t_fast.append(ev[1].elapsed_time(ev[2]))
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        pm, fm = float(np.mean(t_proj)), float(np.mean(t_fast))
        n_proj = n_fast = 1
        schedule = {"kind": "sequential", "streams": 1}
    else:
        # The library's schedule: chunks of C steps, the projection on this
        # stream and the fast matrix on a second one, overlapped.  The timed
        # steps call srdeltanet_forward; then the same schedule is driven chunk
        # by chunk (the same launches, time slices of the same buffers) with
        # HIP events around every launch on its own stream, for the kernels'
        # durations.
        C = srwm.srdeltanet_chunk_steps(w.B, w.T, w.H, w.d_in, w.d_key, w.d_v, w.n_lr)
        aux = torch.cuda.Stream(dev)
        Wc = [torch.empty((w.B, w.H, w.m, w.d_in), dtype=torch.float32, device=dev) for _ in range(2)]
        Fc = [torch.empty((w.B, w.H, w.d_v, w.d_key), dtype=torch.float32, device=dev) for _ in range(2)]

        def step():
            srwm.srdeltanet_forward(x, Wp, w.d_key, w.d_v, apply_input_softmax=w.apply_input_softmax,
                                    n_lr=w.n_lr, z=z, y=y, stream=stream, aux_stream=aux, chunk_steps=C)

        def chunked(t_proj, t_fast):
            for c, t0_ in enumerate(range(0, w.T, C)):
                t1_ = min(w.T, t0_ + C)
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                e[0].record(stream)
                srwm.forward(x[:, t0_:t1_], Wp if c == 0 else Wc[c % 2], apply_input_softmax=w.apply_input_softmax,
                             n_lr=w.n_lr, y=z[:, t0_:t1_], W_T=Wc[(c + 1) % 2], return_state=True, stream=stream)
                e[1].record(stream)
                aux.wait_event(e[1])
                e[2].record(aux)
                srwm.fast_forward(z[:, t0_:t1_], w.d_key, w.d_v, F0=None if c == 0 else Fc[c % 2], y=y[:, t0_:t1_],
                                  F_T=Fc[(c + 1) % 2], stream=aux)
                e[3].record(aux)
                t_proj.append(e[:2])
                t_fast.append(e[2:])
            stream.wait_stream(aux)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps (chunks of {C} steps, two streams)")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t_step = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            ev[0].record(stream)
            step()
            ev[1].record(stream)
            torch.cuda.synchronize()
            t_step.append(ev[0].elapsed_time(ev[1]))
        wall = time.perf_counter() - t0
        ms_per_step = wall * 1e3 / args.steps
        log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step wall, {np.mean(t_step):.3f} ms by events")
        pe, fe = [], []
        for _ in range(args.steps):
            chunked(pe, fe)
        torch.cuda.synchronize()
        n_chunks = (w.T + C - 1) // C
        n_proj = n_fast = n_chunks
        # per step: the sum over its chunk launches
        pm = sum(a.elapsed_time(b) for a, b in pe) / args.steps
        fm = sum(a.elapsed_time(b) for a, b in fe) / args.steps
        schedule = {"kind": "overlapped", "streams": 2, "chunk_steps": C, "chunks": n_chunks,
                    "step_ms_events": float(np.mean(t_step)),
                    "kernel_timing": "the same chunk launches driven one by one, HIP events on each launch's "
                                     "stream"}
    kernels = {
        proj_name: {"ms": pm, "launches_per_step": n_proj, "ms_per_launch": pm / n_proj, "bound": proj_bound,
                    "achieved": proj_flop / (pm * 1e-3) / 1e12, "unit": proj_unit},
        "srwm_fast_kernel": {"ms": fm, "launches_per_step": n_fast, "ms_per_launch": fm / n_fast, "bound": "alu",
                             "achieved": fast_flop / (fm * 1e-3) / 1e12, "unit": "TFLOP/s"},
    }
    for k in kernels.values():
        k["frac"] = k["achieved"] / PEAK_FP32_TFLOPS
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step wall; projection {pm:.3f} ms, fast {fm:.3f} ms "
        f"(kernel time per step)")
    rec = {
        "metric": f"{w.kind} head-steps/sec (B·H·T/s), 1×MI355X",
        "value": w.head_steps / (ms_per_step * 1e-3),
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal x and projection weights; no dataset)",
        "config": {"workload": w.name, "kind": w.kind, "B": w.B, "H": w.H, "d_in": w.d_in, "d_key": w.d_key,
                   "d_v": w.d_v, "T": w.T, "apply_input_softmax": w.apply_input_softmax},
        "roofline": {"bound": kernels[dom]["bound"], "achieved": kernels[dom]["achieved"],
                     "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": kernels[dom]["frac"],
                     "traffic": None, "kernel": dom},
        "kernels": kernels,
        "schedule": schedule,
    }
    if not args.no_cpu:
        from oracle import oracle
        log("[bench] timing the float64 oracle on a bounded sample")
        n = 1
        while True:
            t0 = time.perf_counter()
            xs = np.ascontiguousarray(x_host[:n], dtype=np.float64)
            if w.kind == "deltanet":
                oracle.deltanet_forward(xs, Wp_host, w.d_key, w.d_v)
            else:
                oracle.srdeltanet_forward(xs, Wp_host, w.d_key, w.d_v, apply_input_softmax=w.apply_input_softmax,
                                          n_lr=w.n_lr)
            dt = time.perf_counter() - t0
            if dt * 2 > args.cpu_budget or n >= w.B:
                break
            n = min(w.B, max(n + 1, int(n * min(8.0, args.cpu_budget / max(dt, 1e-3) / 2))))
        rec["cpu_baseline"] = {"value": n * w.H * w.T / dt, "unit": "head-steps/s",
                               "cores": oracle.default_threads(), "kind": "oracle",
                               "sample": f"first {n} of {w.B} sequences x {w.H} heads x T={w.T} of {w.name}, "
                                         f"float64, {dt:.1f} s wall"}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
