"""The five synthetic SRWM workloads and their seeded input generator.

This module holds no arithmetic of the method: it only names shapes and draws
seeded random inputs.  It is the one piece of code that both the GPU path's
tests/bench and the float64 oracle consume.

Input recipe (identical for every consumer):
  * x[b] (shape [T, H, d_in]) is drawn from ``numpy.random.default_rng([seed, 1, b])``
    as float32 standard normals, one independent stream per sequence b, so any
    sampled sequence can be regenerated on its own;
  * W0 (shape [H, m, d_in]) is drawn from ``numpy.random.default_rng([seed, 2])``
    as float64 standard normals scaled by ``w0_std`` and rounded to float32;
  * for bf16 I/O, x is rounded to bfloat16 with round-to-nearest-even; the
    float32 array returned then holds exactly the bf16 values the GPU reads.

Shapes follow the pages' workloads where they give them: 16 heads of width 16
in the sequential multi-task model, input softmax in the RL model (review page
"SRWM: 让权重矩阵学习修改自身", Sec. 2.4 and 3.2-3.3); the larger d and T stress the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d_in: int
    d_out: int
    T: int
    io_dtype: str            # "f32" or "bf16"
    apply_input_softmax: bool
    return_state: bool
    w0_std: float
    seed: int = 0
    n_lr: int = 4            # learning rates: 4 (one per row block) or 1

    @property
    def m(self) -> int:
        return self.d_out + 2 * self.d_in + self.n_lr

    @property
    def units(self) -> int:
        return self.B * self.H

    @property
    def head_steps(self) -> int:
        return self.B * self.H * self.T

    @property
    def flop_per_head_step(self) -> int:
        """Algorithmic work of one head-step: 8*m*d_in (2md projection,
        4md for the two reads, 2md for the rank-one update)."""
        return 8 * self.m * self.d_in

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_d8": Workload("tiny_d8", B=1, H=1, d_in=8, d_out=8, T=16, io_dtype="f32",
                        apply_input_softmax=False, return_state=True, w0_std=0.1),
    "multitask_d16": Workload("multitask_d16", B=4, H=4, d_in=16, d_out=16, T=256,
                              io_dtype="f32", apply_input_softmax=False, return_state=True,
                              w0_std=16 ** -0.5),
    "fewshot_d64": Workload("fewshot_d64", B=32, H=8, d_in=64, d_out=64, T=1024,
                            io_dtype="f32", apply_input_softmax=False, return_state=False,
                            w0_std=64 ** -0.5),
    "rl_d64_bf16": Workload("rl_d64_bf16", B=128, H=16, d_in=64, d_out=64, T=4096,
                            io_dtype="bf16", apply_input_softmax=True, return_state=False,
                            w0_std=64 ** -0.5),
    "wide_d128": Workload("wide_d128", B=8, H=4, d_in=128, d_out=128, T=8192,
                          io_dtype="f32", apply_input_softmax=False, return_state=True,
                          w0_std=128 ** -0.5),
}

#: The workload the headline throughput is quoted on (RL-shaped, d = 64).
HEADLINE = "rl_d64_bf16"


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding the rounded values.  Inputs are finite normals."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def gen_x_seq(w: Workload, b: int, T: int | None = None) -> np.ndarray:
    """x[b] of shape [T, H, d_in] as float32 (bf16-representable for bf16 I/O)."""
    T = w.T if T is None else T
    rng = np.random.default_rng([w.seed, 1, b])
    xb = rng.standard_normal((T, w.H, w.d_in), dtype=np.float32)
    if w.io_dtype == "bf16":
        xb = round_to_bf16(xb)
    return xb


def gen_W0(w: Workload) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 2])
    return (rng.standard_normal((w.H, w.m, w.d_in)) * w.w0_std).astype(np.float32)


def gen_x(w: Workload, batch=None) -> np.ndarray:
    """x[B', T, H, d_in] for the sequences in ``batch`` (default: all B)."""
    bs = range(w.B) if batch is None else list(batch)
    out = np.empty((len(bs), w.T, w.H, w.d_in), dtype=np.float32)
    for i, b in enumerate(bs):
        out[i] = gen_x_seq(w, b)
    return out


def gen_gy(w: Workload, batch=None) -> np.ndarray:
    """Seeded output cotangent gy[B', T, H, d_out] (float32 standard normals),
    one stream per sequence: ``default_rng([seed, 3, b])``."""
    bs = range(w.B) if batch is None else list(batch)
    out = np.empty((len(bs), w.T, w.H, w.d_out), dtype=np.float32)
    for i, b in enumerate(bs):
        out[i] = np.random.default_rng([w.seed, 3, b]).standard_normal((w.T, w.H, w.d_out), dtype=np.float32)
    return out


def gen_gW(w: Workload, batch=None) -> np.ndarray:
    """Seeded final-state cotangent gW_T[B', H, m, d_in] (float32 standard
    normals): ``default_rng([seed, 4, b])``."""
    bs = range(w.B) if batch is None else list(batch)
    out = np.empty((len(bs), w.H, w.m, w.d_in), dtype=np.float32)
    for i, b in enumerate(bs):
        out[i] = np.random.default_rng([w.seed, 4, b]).standard_normal((w.H, w.m, w.d_in), dtype=np.float32)
    return out


# ---------------------------------------------------------------------------
# DeltaNet / SR-DeltaNet workloads (review page Sec. 2.1 and Appendix C.1).
# The pages' RL models use a hidden width of 128 (two heads of 64 here); the
# input recipe is the one above (x per sequence from default_rng([seed, 1, b])),
# DeltaNet's slow projection W_slow[H*P][H*d_in] from default_rng([seed, 5]),
# SR-DeltaNet's SRWM W0[H][m][d_in] from default_rng([seed, 2]); the fast
# matrix starts at zero.
@dataclass(frozen=True)
class FwpWorkload:
    name: str
    kind: str                # "deltanet" or "srdeltanet"
    B: int
    H: int
    d_in: int
    d_key: int
    d_v: int
    T: int
    apply_input_softmax: bool
    w0_std: float
    seed: int = 0
    n_lr: int = 4
    io_dtype: str = "f32"

    @property
    def P(self) -> int:
        """Rows of one head's projection [k; v; q; beta]."""
        return self.d_v + 2 * self.d_key + 1

    @property
    def m(self) -> int:
        """Rows of SR-DeltaNet's SRWM (d_out = P)."""
        return self.P + 2 * self.d_in + self.n_lr

    @property
    def units(self) -> int:
        return self.B * self.H

    @property
    def head_steps(self) -> int:
        return self.B * self.H * self.T

    @property
    def flop_per_head_step(self) -> int:
        """Projection (DeltaNet: 2*P*H*d_in, the full-width product; SR-DeltaNet:
        the SRWM's 8*m*d_in) plus the fast matrix's read, write and query
        (6*d_v*d_key)."""
        proj = 2 * self.P * self.H * self.d_in if self.kind == "deltanet" else 8 * self.m * self.d_in
        return proj + 6 * self.d_v * self.d_key

    def with_(self, **kw) -> "FwpWorkload":
        return replace(self, **kw)


FWP_WORKLOADS = {
    "deltanet_small": FwpWorkload("deltanet_small", "deltanet", B=3, H=2, d_in=16, d_key=16, d_v=16, T=75,
                                  apply_input_softmax=False, w0_std=32 ** -0.5),
    "deltanet_rl": FwpWorkload("deltanet_rl", "deltanet", B=128, H=2, d_in=64, d_key=64, d_v=64, T=4096,
                               apply_input_softmax=False, w0_std=128 ** -0.5),
    "srdeltanet_small": FwpWorkload("srdeltanet_small", "srdeltanet", B=3, H=2, d_in=16, d_key=16, d_v=16,
                                    T=75, apply_input_softmax=True, w0_std=16 ** -0.5),
    "srdeltanet_rl": FwpWorkload("srdeltanet_rl", "srdeltanet", B=128, H=2, d_in=64, d_key=64, d_v=64,
                                 T=4096, apply_input_softmax=True, w0_std=64 ** -0.5),
}


def gen_W_slow(w: FwpWorkload) -> np.ndarray:
    rng = np.random.default_rng([w.seed, 5])
    return (rng.standard_normal((w.H * w.P, w.H * w.d_in)) * w.w0_std).astype(np.float32)
