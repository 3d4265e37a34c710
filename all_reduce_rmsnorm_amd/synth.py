"""Seeded synthetic inputs for the fused epilogue.

This module only draws random numbers and stores them in the tensor formats
the operation consumes (bf16 slabs, residual and gamma).  It holds none of the
operation's arithmetic, so that the GPU path and the CPU oracle can be fed the
same bytes without sharing any of the method's code.

Every tensor has its own stream: ``torch.Generator`` seeded with
``seed * 1000 + stream`` where stream = slab index p (0..P-1) for the per-rank
slabs, 100 for the residual, 200 for gamma and 300 for the outlier mask.  A
value is drawn in fp32 and stored to bf16 by torch's round-to-nearest-even.
"N(0, s)" means ``randn() * s`` (s is the standard deviation).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

STREAM_RESIDUAL = 100
STREAM_GAMMA = 200
STREAM_OUTLIER_MASK = 300


@dataclass(frozen=True)
class Workload:
    """One fused-epilogue (or sum-only) workload: shapes, value laws, scalars."""

    name: str
    P: int
    rows: int
    cols: int
    x_std: float
    residual_std: float | None  # None: no residual
    gamma_law: tuple            # ("uniform", lo, hi) or ("normal", mean, std)
    weight_offset: float = 0.0
    eps: float = 1e-6
    scale_ub: float = 1200.0
    outlier_frac: float = 0.0   # fraction of [rows, cols] positions scaled ...
    outlier_mult: float = 1.0   # ... by this factor, the same positions in every slab
    sum_only: bool = False
    seed: int = 0
    in_place: bool = False      # the residual is updated in place (residual_out == residual_in)
    notes: str = field(default="", compare=False)

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    def algorithmic_bytes(self) -> int:
        """Bytes the operation must move once: P bf16 slabs in, bf16 residual in
        and out (if any), fp8 out, fp32 scales out, bf16 gamma in.  Sum-only:
        P bf16 slabs in, one bf16 tensor out."""
        n = self.numel
        if self.sum_only:
            return 2 * self.P * n + 2 * n
        b = 2 * self.P * n + n + 4 * self.rows + 2 * self.cols
        if self.residual_std is not None:
            b += 4 * n
        return b


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_p2_4x256", P=2, rows=4, cols=256, x_std=1.0, residual_std=None,
                 gamma_law=("uniform", 0.5, 1.5), weight_offset=0.0, eps=1e-6, scale_ub=1200.0),
        Workload("sum_p4_64x4096", P=4, rows=64, cols=4096, x_std=1.0, residual_std=None,
                 gamma_law=("uniform", 1.0, 1.0), sum_only=True),
        Workload("decode_p4_32x7168", P=4, rows=32, cols=7168, x_std=0.5, residual_std=1.0,
                 gamma_law=("uniform", 0.8, 1.2), weight_offset=0.0, eps=1e-6, scale_ub=1200.0,
                 in_place=True, notes="residual updated in place"),
        Workload("unit_offset_p8_128x8192", P=8, rows=128, cols=8192, x_std=0.25, residual_std=1.0,
                 gamma_law=("normal", 0.0, 0.02), weight_offset=1.0, eps=1e-5, scale_ub=1200.0),
        Workload("prefill_p8_8192x7168", P=8, rows=8192, cols=7168, x_std=0.5, residual_std=1.0,
                 gamma_law=("uniform", 0.8, 1.2), weight_offset=0.0, eps=1e-6, scale_ub=64.0,
                 outlier_frac=0.001, outlier_mult=100.0),
        Workload("token_p4_1x7168", P=4, rows=1, cols=7168, x_std=0.5, residual_std=1.0,
                 gamma_law=("uniform", 0.8, 1.2), weight_offset=0.0, eps=1e-6, scale_ub=1200.0,
                 in_place=True, notes="one token with the decode workload's laws; residual updated in place"),
        Workload("token_p8_1x8192", P=8, rows=1, cols=8192, x_std=0.25, residual_std=1.0,
                 gamma_law=("normal", 0.0, 0.02), weight_offset=1.0, eps=1e-5, scale_ub=1200.0,
                 notes="one token with the unit-offset workload's laws"),
        Workload("prefill_share_p8_1024x7168", P=8, rows=1024, cols=7168, x_std=0.5, residual_std=1.0,
                 gamma_law=("uniform", 0.8, 1.2), weight_offset=0.0, eps=1e-6, scale_ub=64.0,
                 outlier_frac=0.001, outlier_mult=100.0,
                 notes="one GPU's row share of the prefill workload on 8 GPUs"),
    ]
}


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def normal_bf16(shape, std, *, seed=0, stream=0, device="cpu", mask=None, mult=1.0):
    """N(0, std) drawn in fp32; positions where ``mask`` is true are multiplied
    by ``mult`` before the value is stored to bf16."""
    x = torch.randn(shape, generator=_gen(device, seed, stream), device=device,
                    dtype=torch.float32) * std
    if mask is not None:
        x = torch.where(mask, x * mult, x)
    return x.to(torch.bfloat16)


def gamma_bf16(cols, law, *, seed=0, device="cpu"):
    g = _gen(device, seed, STREAM_GAMMA)
    if law[0] == "uniform":
        lo, hi = law[1], law[2]
        x = torch.rand((cols,), generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo
    elif law[0] == "normal":
        x = torch.randn((cols,), generator=g, device=device, dtype=torch.float32) * law[2] + law[1]
    else:
        raise ValueError(f"unknown gamma law {law!r}")
    return x.to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", rows: int | None = None, seed: int | None = None):
    """Build ``{'inputs': [P bf16 [rows, cols]], 'residual': bf16 or None, 'gamma': bf16 [cols]}``.

    ``rows`` overrides the workload's row count (for small parity cases with the
    workload's value laws); ``seed`` overrides its seed.
    """
    rows = w.rows if rows is None else rows
    seed = w.seed if seed is None else seed
    shape = (rows, w.cols)
    mask = None
    if w.outlier_frac > 0.0:
        u = torch.rand(shape, generator=_gen(device, seed, STREAM_OUTLIER_MASK), device=device)
        mask = u < w.outlier_frac
    inputs = [normal_bf16(shape, w.x_std, seed=seed, stream=p, device=device, mask=mask,
                          mult=w.outlier_mult) for p in range(w.P)]
    residual = None
    if w.residual_std is not None:
        residual = normal_bf16(shape, w.residual_std, seed=seed, stream=STREAM_RESIDUAL,
                               device=device)
    gamma = gamma_bf16(w.cols, w.gamma_law, seed=seed, device=device)
    return {"inputs": inputs, "residual": residual, "gamma": gamma}


def bf16_bits(t: torch.Tensor):
    """A bf16 tensor's bit patterns as a host numpy uint16 array."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def fp8_bits(t: torch.Tensor):
    """An 8-bit tensor's bit patterns as a host numpy uint8 array."""
    return t.detach().contiguous().cpu().view(torch.uint8).numpy()
