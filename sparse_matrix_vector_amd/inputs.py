"""Seeded synthetic inputs and workload shapes.

Holds none of the method's arithmetic (no pruning, no products): it only
draws random weights and activations, so the GPU path and the CPU oracle can
be fed the same bits.  Recipe:
  * weights: fp32 N(0, 1) * sigma (sigma = 0.02), rounded to fp16/bf16 by
    torch's cast (round to nearest even);
  * activations: N(0, 1), optionally with ceil(1% * K) channels, drawn without
    replacement, scaled by 10 before rounding; or Laplace(0, 1) by inverse CDF;
  * random keep-masks with exactly n kept per m-group (uniform over the
    C(m, n) patterns);
  * every tensor has its own seed, derived from a name by SHA-256, so that a
    tensor can be regenerated alone (on the CPU for small shapes, on the GPU
    for the full-size workloads; the two generators differ, so a test feeds
    both sides from one draw).
"""
import hashlib
import math

import torch

# Projection shapes (R x K = out x in) of the models the pages evaluate.
LLAMA31_8B = {"q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
              "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336)}
LLAMA33_70B = {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
               "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}
QWEN3_14B_MLP = {"gate": (17408, 5120), "up": (17408, 5120), "down": (5120, 17408)}
QWEN3_32B_MLP = {"gate": (25600, 5120), "up": (25600, 5120), "down": (5120, 25600)}
LAYER_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
MLP_ORDER = ("gate", "up", "down")


def seed_of(*parts) -> int:
    """Stable 63-bit seed from a tuple of names/numbers."""
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def weight(R, K, dtype, seed, device="cpu", sigma=0.02):
    g = _gen(seed, device)
    return (torch.randn((R, K), generator=g, device=device, dtype=torch.float32) * sigma).to(dtype)


def activation_normal(B, K, dtype, seed, device="cpu", outlier_frac=0.0, outlier_scale=10.0):
    g = _gen(seed, device)
    x = torch.randn((B, K), generator=g, device=device, dtype=torch.float32)
    if outlier_frac > 0:
        n_out = math.ceil(outlier_frac * K)
        ch = torch.randperm(K, generator=g, device=device)[:n_out]
        x[:, ch] *= outlier_scale
    return x.to(dtype)


def activation_laplace(B, K, dtype, seed, device="cpu"):
    """Laplace(0, 1): x = -sign(u) * ln(1 - 2|u|), u uniform on (-1/2, 1/2)."""
    g = _gen(seed, device)
    u = torch.rand((B, K), generator=g, device=device, dtype=torch.float64) - 0.5
    tail = torch.clamp(1 - 2 * u.abs(), min=2.0 ** -53)
    return (-torch.sign(u) * torch.log(tail)).to(torch.float32).to(dtype)


def keep_mask(R, K, n, m, seed, device="cpu"):
    """uint8 [R][K]: in every m-group exactly n ones, uniform over patterns."""
    g = _gen(seed, device)
    scores = torch.rand((R, K // m, m), generator=g, device=device)
    ranks = scores.argsort(dim=-1).argsort(dim=-1)
    return (ranks < n).to(torch.uint8).reshape(R, K)


def integer_valued(R, K, dtype, seed, lo=-8, hi=8, scale=1.0, device="cpu"):
    """Small integers times a power-of-two scale: every product and partial sum
    of such operands is exact in fp32."""
    g = _gen(seed, device)
    return (torch.randint(lo, hi + 1, (R, K), generator=g, device=device).to(torch.float32) * scale).to(dtype)
