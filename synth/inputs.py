"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module draws random numbers and rounds them to the storage formats the
workloads use. It contains none of the method's arithmetic (no signs, scales,
residuals, packing or products), so that the oracle and the HIP path can both
consume it without sharing any computation.

Workloads (the RaBiT paper, Table 7 and App. E.2, time Llama2 layer shapes;
trained weights are not available, so random-init weights of those shapes
stand in):

* weights  W ~ 0.02 * N(0, 1), float32, row-major [out][in]
* activations x ~ N(0, 1) rounded to bfloat16 (round-to-nearest-even)

Seeds follow one rule everywhere:
  seed_w = 1000 * cfg + 10 * layer + matrix_idx,
  matrix_idx in {q:0, k:1, v:2, o:3, gate:4, up:5, down:6}
  seed_x = 7 + 1000 * cfg + batch
"""
from __future__ import annotations

import numpy as np
import torch

MATRIX_IDX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6}

W_STD = 0.02


def seed_w(cfg: int, layer: int, name: str) -> int:
    return 1000 * cfg + 10 * layer + MATRIX_IDX[name]


def seed_x(cfg: int, batch: int) -> int:
    return 7 + 1000 * cfg + batch


def weight_f32(out: int, inp: int, seed: int, std: float = W_STD,
               device: str = "cpu") -> torch.Tensor:
    """W ~ std * N(0,1) as float32 [out][in], drawn with torch.Generator(seed)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    w = torch.randn(out, inp, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        w.mul_(std)
    return w


def act_bf16(batch: int, inp: int, seed: int, device: str = "cpu") -> torch.Tensor:
    """x ~ N(0,1) rounded to bfloat16, shape [batch][in]."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(batch, inp, generator=g, dtype=torch.float32, device=device)
    return x.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 bit patterns of a bfloat16 CPU tensor."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bfloat16 tensor (bf16 -> f64 is exact)."""
    return t.to(torch.float32).cpu().numpy().astype(np.float64)


def bits_to_bf16_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of raw bfloat16 bit patterns (bf16 is the top half of f32)."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def random_signs(out: int, inp: int, seed: int) -> np.ndarray:
    """Uniform random boolean matrix (True = -1), for layout and pack tests."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2, size=(out, inp), dtype=np.uint8).astype(bool)


def random_f16_scales(n: int, seed: int, lo: float = 0.005, hi: float = 0.03) -> np.ndarray:
    """Positive float16 scale vector (for SCALES_GIVEN tests)."""
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=n).astype(np.float16)


def seed_dy(cfg: int, batch: int) -> int:
    return 53 + 1000 * cfg + batch


def grad_bf16(batch: int, out: int, seed: int, std: float = 0.01,
              device: str = "cpu") -> torch.Tensor:
    """Loss gradient at a layer output, dY ~ std * N(0,1) rounded to bfloat16,
    shape [batch][out] (training-side tests and bench)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    y = torch.randn(batch, out, generator=g, dtype=torch.float32, device=device)
    return y.mul_(std).to(torch.bfloat16)
