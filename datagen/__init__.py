"""Seeded synthetic inputs for the W1.58A8 BitLinear forward.

This module only draws random numbers. It holds none of the method's arithmetic
(no scales, no rounding, no codes): both the CPU oracle and the HIP path receive
exactly the bytes produced here.

Distributions (the shapes and value mixes of the layers the pages describe):

* ``gaussian_weights``  latent fp32 weights ~ N(0, std^2) (std 0.02).
* ``gg_weights``        generalized-Gaussian latents, shape ``beta``; with beta = 0.846
                        the absmean ternary rule yields about 42% zeros and 29% of each
                        sign, the split that "BitNet b1.58 深度解析" (section 2.3) reports
                        for trained weights.
* ``outlier_acts``      activations ~ N(0, 1), each entry independently scaled by 20
                        with probability 0.001.
* ``heavy_channel_acts`` activations ~ N(0, 1), except ceil(0.01 K) channels (chosen by a
                        seeded permutation) that hold Student-t (nu = 3) draws.
* ``gains``             RMSNorm gains ~ U(0.5, 1.5).
* ``bf16_cache``        random bfloat16 bit patterns for a key/value cache: N(0, std^2)
                        draws in binary32 with the low 16 bits dropped.
* ``small_ints``        integers drawn uniformly from [lo, hi], as binary32.

Host generators use numpy's PCG64 seeded through SeedSequence([BASE_SEED, stream]).
``*_torch`` variants draw the same distributions on a torch device (Philox) for
sizes where host generation is too slow; their bytes are copied to the host when
the oracle needs them.
"""
from __future__ import annotations

import math

import numpy as np

BASE_SEED = 0xB17

GG_BETA_TRAINED = 0.846


def stream_id(config: int, layer: int = 0, matrix: int = 0, role: int = 0) -> int:
    """Stream number for one tensor: (config<<16)|(layer<<8)|(matrix<<4)|role."""
    return (config << 16) | (layer << 8) | (matrix << 4) | role


def rng(stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, int(stream)])))


def gaussian_weights(n: int, k: int, stream: int, std: float = 0.02) -> np.ndarray:
    g = rng(stream)
    return (g.standard_normal((n, k), dtype=np.float64) * std).astype(np.float32)


def _gg_scale(beta: float, std: float) -> float:
    # Var of a*sign*G^(1/beta), G ~ Gamma(1/beta): a^2 * Gamma(3/beta) / Gamma(1/beta)
    return std / math.sqrt(math.exp(math.lgamma(3.0 / beta) - math.lgamma(1.0 / beta)))


def gg_weights(n: int, k: int, stream: int, beta: float = GG_BETA_TRAINED,
               std: float = 0.02) -> np.ndarray:
    g = rng(stream)
    a = _gg_scale(beta, std)
    mag = g.standard_gamma(1.0 / beta, size=(n, k)) ** (1.0 / beta)
    sign = np.where(g.random((n, k)) < 0.5, -1.0, 1.0)
    return (a * sign * mag).astype(np.float32)


def outlier_acts(m: int, k: int, stream: int, p: float = 0.001, factor: float = 20.0) -> np.ndarray:
    g = rng(stream)
    x = g.standard_normal((m, k), dtype=np.float64)
    mask = g.random((m, k)) < p
    x = np.where(mask, x * factor, x)
    return x.astype(np.float32)


def heavy_channel_acts(m: int, k: int, stream: int, frac: float = 0.01, nu: float = 3.0) -> np.ndarray:
    g = rng(stream)
    x = g.standard_normal((m, k), dtype=np.float64)
    nheavy = int(math.ceil(frac * k))
    chans = g.permutation(k)[:nheavy]
    x[:, chans] = g.standard_t(nu, size=(m, nheavy))
    return x.astype(np.float32)


def gains(k: int, stream: int) -> np.ndarray:
    g = rng(stream)
    return g.uniform(0.5, 1.5, size=k).astype(np.float32)


def bf16_cache(shape, stream: int, std: float = 1.0) -> np.ndarray:
    g = rng(stream)
    x = (g.standard_normal(shape) * std).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def small_ints(shape, stream: int, lo: int, hi: int) -> np.ndarray:
    return rng(stream).integers(lo, hi + 1, size=shape).astype(np.float32)


# --------------------------------------------------------------------------------------
# Device-side generators (torch, Philox) for full-size workloads.
# --------------------------------------------------------------------------------------

def _torch_gen(stream: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((BASE_SEED << 32) ^ int(stream))
    return gen


def gg_weights_torch(n: int, k: int, stream: int, device, beta: float = GG_BETA_TRAINED,
                     std: float = 0.02):
    """GG(beta) latents drawn on ``device``; returns a contiguous fp32 tensor [n][k]."""
    import torch
    gen = _torch_gen(stream, device)
    a = _gg_scale(beta, std)
    alpha = torch.full((n, k), 1.0 / beta, dtype=torch.float32, device=device)
    mag = torch._standard_gamma(alpha, generator=gen)
    del alpha
    mag.pow_(1.0 / beta)
    u = torch.rand((n, k), generator=gen, dtype=torch.float32, device=device)
    mag.mul_(torch.where(u < 0.5, -a, a))
    return mag.contiguous()


def gaussian_weights_torch(n: int, k: int, stream: int, device, std: float = 0.02):
    import torch
    gen = _torch_gen(stream, device)
    w = torch.randn((n, k), generator=gen, dtype=torch.float32, device=device)
    return w.mul_(std)


def outlier_acts_torch(m: int, k: int, stream: int, device, p: float = 0.001, factor: float = 20.0):
    import torch
    gen = _torch_gen(stream, device)
    x = torch.randn((m, k), generator=gen, dtype=torch.float32, device=device)
    u = torch.rand((m, k), generator=gen, dtype=torch.float32, device=device)
    return torch.where(u < p, x * factor, x).contiguous()


def heavy_channel_acts_torch(m: int, k: int, stream: int, device, frac: float = 0.01, nu: float = 3.0):
    import torch
    gen = _torch_gen(stream, device)
    x = torch.randn((m, k), generator=gen, dtype=torch.float32, device=device)
    nheavy = int(math.ceil(frac * k))
    chans = torch.randperm(k, generator=gen, device=device)[:nheavy]
    z = torch.randn((m, nheavy), generator=gen, dtype=torch.float32, device=device)
    chi2 = 2.0 * torch._standard_gamma(torch.full((m, nheavy), nu / 2.0, device=device), generator=gen)
    x[:, chans] = z / torch.sqrt(chi2 / nu)
    return x.contiguous()


def gains_torch(k: int, stream: int, device):
    import torch
    gen = _torch_gen(stream, device)
    return (torch.rand((k,), generator=gen, dtype=torch.float32, device=device) + 0.5).contiguous()
