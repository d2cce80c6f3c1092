"""bench.py end to end on the GPU (short runs): one JSON line with the fields
its readers rely on, for the forward headline (with the CPU oracle baseline)
and the training step."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]


def bench(args):
    r = subprocess.run([sys.executable, "-u", str(ROOT / "bench.py"), *args], capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_common(d, metric_word):
    assert metric_word in d["metric"]
    assert d["value"] > 0 and d["unit"] == "head-steps/s"
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["dtype"] == "f32" and "synthetic" in d["data"]
    assert d["ms_per_step"] > 0 and d["config"]["workload"].startswith("rl_d64_bf16")
    rf = d["roofline"]
    assert rf["bound"] == "alu" and rf["unit"] == "TFLOP/s" and rf["peak"] == pytest.approx(157.3)
    assert 0 < rf["frac"] < 1 and rf["achieved"] == pytest.approx(rf["frac"] * rf["peak"])


def test_forward_line():
    d = bench(["--steps", "3", "--warmup", "1", "--cpu-budget", "2", "--config-cpu-budget", "1"])
    check_common(d, "head-steps/sec")
    # B*H*T / time per step
    assert d["value"] == pytest.approx(128 * 16 * 4096 / (d["ms_per_step"] * 1e-3), rel=1e-6)
    assert d["kernel"]["resources"]["vgprs"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == "head-steps/s"
    assert cb["sample"] and cb["cpu_model"]
    assert cb["threads"] == cb["cores"] and cb["affinity_cpus"] >= 1
    # the chip's measured LDS read bandwidth, and the five workloads
    assert d["calibration"]["lds"]["lds_read_TBps"] > 0
    from self_referential_weight_amd.workloads import WORKLOADS
    assert set(d["configs"]) == set(WORKLOADS)
    for name, c in d["configs"].items():
        w = WORKLOADS[name]
        assert c["launches"] >= 3 and 0 < c["ms_min"] <= c["ms_median"]
        assert c["head_steps_per_s"] == pytest.approx(w.head_steps / (c["ms_median"] * 1e-3))
        assert c["executed_frac"] == pytest.approx(0.75 * c["frac"]) and 0 < c["frac"] < 1
        assert c["cpu_baseline"]["kind"] == "oracle" and c["cpu_baseline"]["value"] > 0
    assert d["configs"]["rl_d64_bf16"]["cpu_baseline"] == cb


def test_training_line():
    d = bench(["--backward", "--steps", "2", "--warmup", "1", "--no-cpu"])
    check_common(d, "training")
    assert d["forward_ms"] > 0 and d["backward_ms"] > 0
    assert d["backward_kernel_resources"]["threads"] == 256
