"""Seeded synthetic workloads for the MoE layer with zero-computation experts.

This module only draws random numbers: it holds none of the layer's
arithmetic.  Both the HIP library (through the tests and the benchmark) and
the CPU oracle are fed from the tensors it returns, so the two sides always
see the same, already rounded, input values.

Shapes follow the LongCat-Flash layer ("LongCat-Flash Technical Report",
section 2.4 "Model information": hidden size 6144, 512 FFN experts with
inner size 2048, 256 zero-computation experts, 12 experts per token) and
four smaller variants of it.  Every tensor has its own generator stream:
    seed = 1_000_000 * config_id + 10_000 * tensor_code + expert
with tensor codes 1 x, 2 router weight, 3 gate weight, 4 up weight,
5 down weight, 6 bias, 7 output gradient, 8 Zipf rank permutation.  Per-step
training inputs use 100_000_000 + 1000 * step + code (1 for x, 7 for dY).
Values are drawn in fp32 (N(0, std) means standard deviation std) and then
rounded to nearest-even bf16 for the bf16 workloads.

Generators on "cpu" and "cuda" produce different streams for the same seed;
callers pick one device per workload and copy the result to the other side.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class LayerShape:
    name: str
    cid: int          # config id, part of every seed
    T: int            # tokens
    d: int            # hidden size
    N: int            # FFN experts
    Z: int            # zero-computation (identity) experts
    I: int            # FFN inner size
    K: int            # experts per token
    dtype: str        # "f32" or "bf16" (x, weights, outputs)
    w_std: float      # std of every weight matrix
    bias: str         # "zero", "uniform" (U(-0.1, 0.1)), "zipf"
    forward_only: bool = True

    @property
    def E(self) -> int:
        return self.N + self.Z

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_T(self, T: int) -> "LayerShape":
        return replace(self, T=T)


CONFIGS = {
    "tiny_fp32": LayerShape("tiny_fp32", 1, 64, 128, 8, 4, 64, 2, "f32", 0.02, "zero"),
    "small_bf16": LayerShape("small_bf16", 2, 4096, 1024, 64, 32, 512, 6, "bf16", 0.02,
                             "uniform"),
    "decode_bf16": LayerShape("decode_bf16", 3, 256, 6144, 512, 256, 2048, 12, "bf16",
                              0.006, "zero"),
    "prefill_bf16": LayerShape("prefill_bf16", 4, 16384, 6144, 512, 256, 2048, 12, "bf16",
                               0.006, "zipf"),
    "train_bf16": LayerShape("train_bf16", 5, 8192, 2048, 128, 64, 1024, 8, "bf16", 0.02,
                             "zero", forward_only=False),
}

# Zipf-ranked bias for the skewed prefill workload: the FFN expert of rank r
# (1-based, ranks assigned by a seeded permutation) gets ZIPF_B0 * r**-ZIPF_S;
# zero-computation experts get 0.
ZIPF_B0 = 0.005
ZIPF_S = 1.1
# Training loop: expected number of FFN experts per token and adaptation rate.
TRAIN_K_E = 6.0
TRAIN_MU = 1.0
TRAIN_STEPS = 50
# Device-level load-balance loss of the training layer: its 128 FFN experts
# in 8 groups of 16 (one group per device of an 8-way expert-parallel
# placement); the balance factor is not printed with the loss, 1e-3 is a
# stated choice.
TRAIN_LB_D = 8
TRAIN_LB_ALPHA = 1e-3

X, WR, WG, WU, WD, BIAS, DY, RANK = 1, 2, 3, 4, 5, 6, 7, 8


def seed(cid: int, code: int, e: int = 0) -> int:
    return 1_000_000 * cid + 10_000 * code + e


def step_seed(step: int, code: int) -> int:
    return 100_000_000 + 1000 * step + code


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def normal(shape, std, s, device, dtype) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, s), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def make_bias(shape: LayerShape, device="cpu") -> torch.Tensor:
    E, N = shape.E, shape.N
    if shape.bias == "zero":
        return torch.zeros(E, dtype=torch.float32, device=device)
    if shape.bias == "uniform":
        g = _gen("cpu", seed(shape.cid, BIAS))
        b = torch.rand(E, generator=g, dtype=torch.float32) * 0.2 - 0.1
        return b.to(device)
    if shape.bias == "zipf":
        g = _gen("cpu", seed(shape.cid, RANK))
        rank = torch.randperm(N, generator=g) + 1
        b = torch.zeros(E, dtype=torch.float64)
        b[:N] = ZIPF_B0 * rank.double() ** (-ZIPF_S)
        return b.float().to(device)
    raise ValueError(shape.bias)


def make_layer(shape: LayerShape, device="cpu", want_experts=True) -> dict:
    """x [T,d], wr [E,d], wg/wu [N,I,d], wd [N,d,I], bias [E] fp32."""
    dt, c = shape.torch_dtype, shape.cid
    T, d, N, I, E = shape.T, shape.d, shape.N, shape.I, shape.E
    out = {
        "x": normal((T, d), 1.0, seed(c, X), device, dt),
        "wr": normal((E, d), shape.w_std, seed(c, WR), device, dt),
        "bias": make_bias(shape, device),
    }
    if want_experts:
        wg = torch.empty((N, I, d), dtype=dt, device=device)
        wu = torch.empty((N, I, d), dtype=dt, device=device)
        wd = torch.empty((N, d, I), dtype=dt, device=device)
        for e in range(N):
            wg[e] = normal((I, d), shape.w_std, seed(c, WG, e), device, dt)
            wu[e] = normal((I, d), shape.w_std, seed(c, WU, e), device, dt)
            wd[e] = normal((d, I), shape.w_std, seed(c, WD, e), device, dt)
        out.update(wg=wg, wu=wu, wd=wd)
    return out


def make_dy(shape: LayerShape, device="cpu") -> torch.Tensor:
    return normal((shape.T, shape.d), 1.0, seed(shape.cid, DY), device, shape.torch_dtype)


def step_x(shape: LayerShape, step: int, device="cpu") -> torch.Tensor:
    return normal((shape.T, shape.d), 1.0, step_seed(step, X), device, shape.torch_dtype)


def step_dy(shape: LayerShape, step: int, device="cpu") -> torch.Tensor:
    return normal((shape.T, shape.d), 1.0, step_seed(step, DY), device, shape.torch_dtype)


def make_logits(T: int, E: int, std: float, s: int, device="cpu") -> torch.Tensor:
    """Stand-alone fp32 router scores, for routing fed with given logits."""
    return normal((T, E), std, s, device, torch.float32)


def to_np(t: torch.Tensor) -> np.ndarray:
    """Host numpy view for the oracle: fp32 stays fp32, bf16 becomes its
    16-bit pattern (uint16); other dtypes keep their numpy type."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)
