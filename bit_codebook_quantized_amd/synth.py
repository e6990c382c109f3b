"""Seeded synthetic inputs for the ConvRot W4A8 layer (tests, bench, smoke).

This module holds none of the layer's arithmetic: it draws random numbers,
rounds fp32 draws to bfloat16 with torch's own conversion, and draws random
storage bytes.  Both the HIP path and the CPU oracle consume what it returns;
neither is imported here.

Seed recipe: ``seed_for(config, layer, role)`` = 1_000_000*config + 1000*layer
+ role, with role 0 = weight, 1 = activation, 2 = outlier-column choice,
3 = random storage bytes.  Generator: NumPy PCG64.
"""

from __future__ import annotations

import numpy as np

ROLE_WEIGHT, ROLE_ACT, ROLE_OUTLIER, ROLE_BYTES = 0, 1, 2, 3


def seed_for(config: int, layer: int = 0, role: int = 0) -> int:
    return 1_000_000 * config + 1000 * layer + role


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """fp32 draws -> the nearest bfloat16 values, returned as fp32 (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.to(torch.float32).numpy()


def gaussian_weight(n: int, k: int, seed: int, std: float = 0.02) -> np.ndarray:
    """fp32 weight [n, k] with i.i.d. N(0, std^2) entries."""
    return (rng(seed).standard_normal((n, k)) * std).astype(np.float32)


def gaussian_weight_device(n: int, k: int, seed: int, device, std: float = 0.02):
    """fp32 torch tensor [n, k] of i.i.d. N(0, std^2) entries drawn on ``device`` by
    torch's generator seeded with ``seed`` (a different stream from gaussian_weight;
    for large benchmark weight sets that would be slow to draw on the host)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std


def activations_device(m: int, k: int, seed: int, device):
    """bf16 torch tensor [m, k] of N(0, 1) draws made on ``device`` by torch's generator
    seeded with ``seed`` (for large benchmark activations; a different stream from
    ``activations``)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(m, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def activations(m: int, k: int, seed: int, kind: str = "normal", nu: float = 4.0,
                outlier_frac: float = 0.01, outlier_scale: float = 20.0,
                outlier_seed: int | None = None) -> np.ndarray:
    """bf16-valued activations [m, k] (as fp32).

    kind 'normal': N(0, 1).  kind 'student_t': standard Student-t with ``nu``
    degrees of freedom.  kind 'outliers': N(0, 1) with round(outlier_frac * k)
    columns, chosen without replacement by a generator seeded with
    ``outlier_seed``, multiplied by ``outlier_scale`` in fp32.  The single
    rounding to bf16 happens last."""
    g = rng(seed)
    if kind == "normal":
        x = g.standard_normal((m, k)).astype(np.float32)
    elif kind == "student_t":
        x = g.standard_t(nu, size=(m, k)).astype(np.float32)
    elif kind == "outliers":
        x = g.standard_normal((m, k)).astype(np.float32)
        n_out = int(round(outlier_frac * k))
        cols = rng(outlier_seed if outlier_seed is not None else seed + 1).choice(k, size=n_out, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    else:
        raise ValueError(kind)
    return to_bf16_values(x)


def random_layer_bytes(n: int, k: int, seed: int, group: int = 16,
                       srel_lo: int = 0x00, srel_hi: int = 0xFF):
    """A packed layer of random storage: codes uniform in 0..15 (two per byte),
    relative-scale bytes uniform in [srel_lo, srel_hi] (all 256 bytes by
    default, NaN patterns included), and positive fp32 channel scales.
    Returns (packed u8 [n, k/2], srel u8 [n, k/group], s_channel fp32 [n])."""
    g = rng(seed)
    packed = g.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    srel = g.integers(srel_lo, srel_hi + 1, size=(n, k // group), dtype=np.int64).astype(np.uint8)
    s_channel = (g.uniform(0.5, 2.0, size=n) * 2e-4).astype(np.float32)
    return packed, srel, s_channel
