"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds only random-number generation and dtype casts of the
generated values; it contains none of the quantization or matmul arithmetic.
Values follow the workloads the pages describe: activations ~N(0, 1); weights
~N(0, 0.02) (or ~N(0, 1) for the tiny case, as in the MLX issue #4720
reproducer); an outlier variant scales a random 1% of weights by 20.
Generation happens in fp32 and is then cast (round-to-nearest-even) to the
activation dtype.
"""

from __future__ import annotations

import numpy as np
import torch

TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def seed_for(config: int, role: int, index: int) -> int:
    """Seed recipe: 1000*config + 10*role + index (role 0 = W, 1 = x, 2 = outlier mask)."""
    return 1000 * config + 10 * role + index


def normal(shape, std: float, dt: str, seed: int, device="cpu",
           outlier_frac: float = 0.0, outlier_scale: float = 20.0) -> torch.Tensor:
    """N(0, std^2) values in fp32, optional outliers, cast to ``dt``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    v = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * std
    if outlier_frac > 0:
        g2 = torch.Generator(device=device)
        g2.manual_seed(int(seed) + 7919)
        mask = torch.rand(tuple(shape), generator=g2, device=device) < outlier_frac
        v = torch.where(mask, v * outlier_scale, v)
    return v.to(TORCH_DT[dt])


def to_oracle(t: torch.Tensor) -> np.ndarray:
    """Host numpy view used by the oracle: fp16 -> float16, bf16 -> uint16 bits."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float16:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def from_oracle(a: np.ndarray, dt: str | None = None) -> torch.Tensor:
    """Inverse of :func:`to_oracle` (host tensor)."""
    if a.dtype == np.float16:
        return torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        assert dt == "bf16"
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32))
    return torch.from_numpy(np.ascontiguousarray(a))


def special_groups(kind: str, N: int, K: int, gs: int, dt: str, seed: int) -> torch.Tensor:
    """Structured weight rows for edge cases.

    kind: "constant" (every group constant), "tiny" (groups spanning a few
    ulps around a random centre), "mixed" (random mix of constant, tiny,
    normal and outlier groups).
    """
    rng = np.random.default_rng(seed)
    G = K // gs
    if kind == "constant":
        c = rng.standard_normal((N, G, 1)).astype(np.float32)
        v = np.broadcast_to(c, (N, G, gs)).copy()
    elif kind == "tiny":
        c = rng.standard_normal((N, G, 1)).astype(np.float32)
        jitter = rng.integers(-3, 4, size=(N, G, gs)).astype(np.float32)
        v = c * (1.0 + jitter * np.float32(2.0 ** -9))
    elif kind == "mixed":
        v = rng.standard_normal((N, G, gs)).astype(np.float32) * 0.02
        pick = rng.integers(0, 4, size=(N, G))
        c = rng.standard_normal((N, G, 1)).astype(np.float32)
        v = np.where((pick == 0)[..., None], c, v)
        v = np.where((pick == 1)[..., None], c * (1 + rng.integers(-2, 3, size=(N, G, gs)) * 2.0 ** -9), v)
        big = rng.random((N, G, gs)) < 0.05
        v = np.where((pick == 3)[..., None] & big, v * 20, v)
    else:
        raise ValueError(kind)
    return torch.from_numpy(np.ascontiguousarray(v.reshape(N, K).astype(np.float32))).to(TORCH_DT[dt])
