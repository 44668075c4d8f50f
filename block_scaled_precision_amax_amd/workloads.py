"""Seeded synthetic inputs for the FP8 quantize / block-scaled GEMM path.

Only random-number generation and input construction lives here (no
quantization or GEMM arithmetic), so the tests can hand the same bytes to
the GPU library and to the CPU oracle, and the benchmark can build its
workloads.  Every generator takes a seed and a device; the same seed on
the same device gives the same bytes.

The recipes follow the workloads of the source pages:
  * the outlier experiment of the handbook chapter "混合精度与 FP8 训练",
    section "FP8 训练": a 256x1024 fp32 N(0,1) activation whose columns
    0-3 are multiplied by an outlier factor;
  * activations N(0,1) with a few outlier channels (columns), weights
    0.02*N(0,1) stored [out, in] as nn.Linear does (PyTorch-native FP8
    article, section 3.1), gradients with magnitudes spread from 1e-6 to
    1e-2 (the same article, section 1.2: gradients jump between 1e-2 and
    1e-6);
  * a delayed-scaling sequence whose per-step spread drifts
    log-uniformly between 0.5 and 50.
"""
from __future__ import annotations

import math

import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, device="cpu", std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    x = torch.randn(*shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def activation(rows: int, cols: int, seed: int, device="cpu", outlier_cols: int = 4,
               factor: float = 1e4, dtype=torch.float32) -> torch.Tensor:
    """N(0,1) activations whose first `outlier_cols` columns are scaled by `factor`."""
    x = torch.randn(rows, cols, generator=_gen(seed, device), device=device, dtype=torch.float32)
    if outlier_cols:
        x[:, :outlier_cols] *= factor
    return x.to(dtype)


def weight(out_features: int, in_features: int, seed: int, device="cpu", std: float = 0.02,
           dtype=torch.float32) -> torch.Tensor:
    """std*N(0,1) weight stored [out, in] (K-contiguous)."""
    return normal((out_features, in_features), seed, device, std, dtype)


def gradient(rows: int, cols: int, seed: int, device="cpu", lo: float = 1e-6, hi: float = 1e-2,
             dtype=torch.float32) -> torch.Tensor:
    """Random-sign values with |g| log-uniform in [lo, hi]."""
    g = _gen(seed, device)
    u = torch.rand(rows, cols, generator=g, device=device, dtype=torch.float32)
    sign = torch.randint(0, 2, (rows, cols), generator=g, device=device, dtype=torch.int8)
    mag = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    mag = torch.where(sign == 1, -mag, mag)
    return mag.to(dtype)


def sigma_schedule(steps: int, seed: int, lo: float = 0.5, hi: float = 50.0) -> list[float]:
    """Per-step spread sigma_t = lo * (hi/lo)^u_t with u_t ~ U[0,1) i.i.d."""
    g = _gen(seed, "cpu")
    u = torch.rand(steps, generator=g, dtype=torch.float64)
    return [float(lo * (hi / lo) ** v) for v in u]


def delayed_step(rows: int, cols: int, sigma: float, seed: int, device="cpu",
                 dtype=torch.bfloat16) -> torch.Tensor:
    """One step's tensor of the delayed-scaling sequence: sigma * N(0,1)."""
    return normal((rows, cols), seed, device, sigma, dtype)


def fp8_codes(shape, fmt: int, seed: int, device="cpu") -> torch.Tensor:
    """Uniformly random finite FP8 codes of format fmt (0 = E4M3FN, 1 = E5M2)."""
    g = _gen(seed, device)
    c = torch.randint(0, 256, shape, generator=g, device=device, dtype=torch.int32)
    if fmt == 0:  # 0x7F / 0xFF are the only non-finite E4M3FN codes
        c = torch.where((c & 0x7F) == 0x7F, c - 1, c)
    else:  # E5M2 exponent 31 holds Inf / NaN
        c = torch.where((c & 0x7F) >= 0x7C, c & 0xFB, c)
    return c.to(torch.uint8)


def to_bits_u16(x: torch.Tensor):
    """Raw bf16 bits of a bf16 tensor as a numpy uint16 array (CPU copy)."""
    import numpy as np

    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_numpy_input(x: torch.Tensor):
    """A CPU numpy view of an fp32 tensor, or the raw bits of a bf16 one."""
    if x.dtype == torch.bfloat16:
        return to_bits_u16(x)
    return x.detach().cpu().contiguous().numpy()
