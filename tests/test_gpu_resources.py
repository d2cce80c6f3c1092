"""Registers, LDS, scratch and occupancy that the HIP runtime reports for the
kernels (the figures bench.py puts in its JSON line), checked against what the
kernels are built for."""
import pytest

import self_referential_weight_amd as srwm
from self_referential_weight_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu


def test_forward_variants_resources():
    for v in srwm.variants():
        r = srwm.kernel_resources(v["index"])
        assert r["threads"] == 64 * v["waves"]
        assert 0 < r["vgprs"] <= 512
        assert r["lds_bytes"] > 0
        assert r["scratch_bytes"] >= 0
        assert r["workgroups_per_cu"] >= 1
        # the occupancy each variant is built for is reached (its registers and
        # LDS allow it), and a workgroup's waves spread over the four SIMDs
        assert r["waves_per_simd"] >= max(v["waves_per_simd"], -(-v["waves"] // 4)), (v, r)


def test_headline_kernel_occupancy():
    w = WORKLOADS["rl_d64_bf16"]
    v = srwm.select_variant(w.d_in, w.d_out, w.io_dtype, w.units)
    r = srwm.kernel_resources(v["index"])
    # one wave per unit, two waves per SIMD: all 2048 units resident on 256 CUs
    assert v["waves"] == 1 and r["waves_per_simd"] >= 2
    assert r["workgroups_per_cu"] * 256 >= w.units


def test_backward_resources():
    for d in (8, 16, 64, 128):
        for n_lr in (4, 1):
            r = srwm.backward_resources(d, d, n_lr, False)
            assert 0 < r["vgprs"] <= 512 and r["workgroups_per_cu"] >= 1
            if d != 128:
                assert srwm.backward_resources(d, d, n_lr, True)["threads"] == r["threads"]
    # d = 64: four waves per unit when there are enough units, eight below
    r = srwm.backward_resources(64, 64, 4, False, 2048)
    assert r["threads"] == 256 and r["waves_per_simd"] == 2
    assert srwm.backward_resources(64, 64, 4, False, 256)["threads"] == 512
