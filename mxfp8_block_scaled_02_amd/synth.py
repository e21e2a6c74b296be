"""Seeded synthetic inputs for the five MXFP8 workloads.

This module only draws random numbers and rounds them to bf16; it holds none
of the quantization arithmetic, so both the GPU library's tests and the CPU
oracle can consume its output.  Every tensor is produced in float32 from a
``torch.Generator`` seeded per workload (1000 + workload number) and rounded
to bf16 by torch (round to nearest even).  With ``device="cuda"`` the draws
come from the device generator (different numbers, same recipe); callers that
compare against the oracle copy the device bytes back, so both sides always
see the same input.

Workloads (sizes are one GPU's share at its real shape):

1. rowwise quantize of x [256, 1024] ~ N(0, 1)
2. rowwise + columnwise quantize of a weight [4096, 4096] ~ N(0, 0.02), with
   0.1% of elements scaled x1000, 1% of the aligned 32x32 tiles all zero and
   another, disjoint 1% holding bf16 subnormals (exponent field 0, mantissa
   uniform in 1..127, random sign)
3. RMSNorm + rowwise quantize of x [8192, 8192] ~ N(0, 1), gamma [8192] ~
   N(1, 0.1), weight offset 1.0, eps 1e-6
4. grouped rowwise + columnwise quantize of 64 expert weights [2048, 7168] ~
   N(0, 0.01)
5. RMSNorm + rowwise quantize at decode [16, 7168] and prefill [65536, 7168]:
   x = N(0, 3) * 10^u with u ~ U(-2, 2) drawn once per row, gamma ~ N(1, 0.1),
   offset 0.0, eps 1e-5
6. rowwise + columnwise quantize of a float32 master weight [4096, 4096]: the
   recipe of 2 kept in float32, with float32 subnormal tiles
7. rowwise-only quantize of a prefill activation [8192, 7168] ~ N(0, 1): the
   activation a linear layer quantizes before its MXFP8 product
"""
from __future__ import annotations

import torch

TILE = 32  # side of the aligned tiles that the zero / subnormal recipe selects

SHAPES = {
    "rowwise_256x1024": (256, 1024),
    "rowcol_4096x4096": (4096, 4096),
    "rmsnorm_8192x8192": (8192, 8192),
    "grouped_64x2048x7168": (64, 2048, 7168),
    "rmsnorm_decode_16x7168": (16, 7168),
    "rmsnorm_prefill_65536x7168": (65536, 7168),
    "rowcol_f32_4096x4096": (4096, 4096),
    "rowwise_8192x7168": (8192, 7168),
}
SEEDS = {
    "rowwise_256x1024": 1001,
    "rowcol_4096x4096": 1002,
    "rmsnorm_8192x8192": 1003,
    "grouped_64x2048x7168": 1004,
    "rmsnorm_decode_16x7168": 1005,
    "rmsnorm_prefill_65536x7168": 1005,
    "rowcol_f32_4096x4096": 1006,
    "rowwise_8192x7168": 1007,
}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, std: float, gen: torch.Generator, mean: float = 0.0,
                device="cpu") -> torch.Tensor:
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (x * std + mean).to(torch.bfloat16)


def rowwise_input(rows=256, cols=1024, seed=1001, device="cpu") -> torch.Tensor:
    g = generator(seed, device)
    return normal_bf16((rows, cols), 1.0, g, device=device)


def weight_with_outliers(rows=4096, cols=4096, seed=1002, device="cpu",
                         std=0.02, outlier_frac=0.001, outlier_gain=1000.0,
                         zero_tile_frac=0.01, subnormal_tile_frac=0.01) -> torch.Tensor:
    """The rowwise + columnwise weight recipe (see the module docstring)."""
    g = generator(seed, device)
    n = rows * cols
    x = torch.randn((n,), generator=g, device=device, dtype=torch.float32) * std
    n_out = int(round(outlier_frac * n))
    if n_out:
        idx = torch.randperm(n, generator=g, device=device)[:n_out]
        x[idx] *= outlier_gain
    x = x.to(torch.bfloat16).view(rows, cols)
    bits = x.view(torch.int16)
    tr, tc = rows // TILE, cols // TILE
    n_tiles = tr * tc
    n_zero = int(round(zero_tile_frac * n_tiles))
    n_sub = int(round(subnormal_tile_frac * n_tiles))
    if n_tiles and (n_zero or n_sub):
        pick = torch.randperm(n_tiles, generator=g, device=device)[: n_zero + n_sub]
        for k, t in enumerate(pick.tolist()):
            r0, c0 = (t // tc) * TILE, (t % tc) * TILE
            if k < n_zero:
                bits[r0:r0 + TILE, c0:c0 + TILE] = 0
            else:
                mant = torch.randint(1, 128, (TILE, TILE), generator=g, device=device,
                                     dtype=torch.int32)
                sign = torch.randint(0, 2, (TILE, TILE), generator=g, device=device,
                                     dtype=torch.int32)
                # bf16 subnormal: exponent field 0, mantissa 1..127, any sign
                pattern = (sign << 15) | mant
                pattern = torch.where(pattern >= 0x8000, pattern - 0x10000, pattern)
                bits[r0:r0 + TILE, c0:c0 + TILE] = pattern.to(torch.int16)
    return x


def master_weight_f32(rows=4096, cols=4096, seed=1006, device="cpu", std=0.02,
                      outlier_frac=0.001, outlier_gain=1000.0, zero_tile_frac=0.01,
                      subnormal_tile_frac=0.01) -> torch.Tensor:
    """The weight recipe kept in float32 (a master weight): N(0, std) with
    outliers, all-zero 32x32 tiles and tiles of float32 subnormals (exponent
    field 0, random mantissa and sign)."""
    g = generator(seed, device)
    n = rows * cols
    x = torch.randn((n,), generator=g, device=device, dtype=torch.float32) * std
    n_out = int(round(outlier_frac * n))
    if n_out:
        idx = torch.randperm(n, generator=g, device=device)[:n_out]
        x[idx] *= outlier_gain
    x = x.view(rows, cols)
    bits = x.view(torch.int32)
    tr, tc = rows // TILE, cols // TILE
    n_tiles = tr * tc
    n_zero = int(round(zero_tile_frac * n_tiles))
    n_sub = int(round(subnormal_tile_frac * n_tiles))
    if n_tiles and (n_zero or n_sub):
        pick = torch.randperm(n_tiles, generator=g, device=device)[: n_zero + n_sub]
        for k, t in enumerate(pick.tolist()):
            r0, c0 = (t // tc) * TILE, (t % tc) * TILE
            if k < n_zero:
                bits[r0:r0 + TILE, c0:c0 + TILE] = 0
            else:
                mant = torch.randint(1, 1 << 23, (TILE, TILE), generator=g, device=device,
                                     dtype=torch.int32)
                sign = torch.randint(0, 2, (TILE, TILE), generator=g, device=device,
                                     dtype=torch.int32)
                bits[r0:r0 + TILE, c0:c0 + TILE] = mant | (sign << 31)
    return x


def rmsnorm_inputs(rows, cols, seed, device="cpu", x_std=1.0, row_decades=0.0,
                   gamma_std=0.1):
    """(x, gamma): x ~ N(0, x_std) times 10^u per row with u ~ U(-d, d), gamma ~ N(1, gamma_std)."""
    g = generator(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32) * x_std
    if row_decades:
        u = (torch.rand((rows, 1), generator=g, device=device, dtype=torch.float32) * 2 - 1)
        x = x * torch.pow(10.0, u * row_decades)
    gamma = torch.randn((cols,), generator=g, device=device, dtype=torch.float32)
    gamma = gamma * gamma_std + 1.0
    return x.to(torch.bfloat16), gamma.to(torch.bfloat16)


def expert_weights(n=64, rows=2048, cols=7168, seed=1004, device="cpu", std=0.01):
    """List of n expert weights [rows, cols] ~ N(0, std), drawn one after another."""
    g = generator(seed, device)
    return [normal_bf16((rows, cols), std, g, device=device) for _ in range(n)]


def workload(name: str, device="cpu", **overrides):
    """Inputs of a named workload as a dict of tensors and scalars."""
    seed = overrides.pop("seed", SEEDS[name])
    if name in ("rowwise_256x1024", "rowwise_8192x7168"):
        r, c = overrides.get("shape", SHAPES[name])
        return {"x": rowwise_input(r, c, seed, device)}
    if name == "rowcol_4096x4096":
        r, c = overrides.get("shape", SHAPES[name])
        return {"x": weight_with_outliers(r, c, seed, device)}
    if name == "rmsnorm_8192x8192":
        r, c = overrides.get("shape", SHAPES[name])
        x, gamma = rmsnorm_inputs(r, c, seed, device, x_std=1.0)
        return {"x": x, "gamma": gamma, "weight_offset": 1.0, "eps": 1e-6}
    if name == "grouped_64x2048x7168":
        n, r, c = overrides.get("shape", SHAPES[name])
        return {"xs": expert_weights(n, r, c, seed, device)}
    if name == "rowcol_f32_4096x4096":
        r, c = overrides.get("shape", SHAPES[name])
        return {"x": master_weight_f32(r, c, seed, device)}
    if name in ("rmsnorm_decode_16x7168", "rmsnorm_prefill_65536x7168"):
        r, c = overrides.get("shape", SHAPES[name])
        x, gamma = rmsnorm_inputs(r, c, seed, device, x_std=3.0, row_decades=2.0)
        return {"x": x, "gamma": gamma, "weight_offset": 0.0, "eps": 1e-5}
    raise KeyError(name)


def bf16_bits(t: torch.Tensor):
    """uint16 numpy view of a bf16 tensor's bit patterns (copied to host)."""
    import numpy as np
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
