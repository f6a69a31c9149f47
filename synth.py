"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and nothing else: it holds none of the
quantisation, normalisation or GEMM arithmetic. Every tensor is drawn on the
CPU from a seeded ``torch.Generator`` as fp32 ``randn * sigma`` and rounded to
BF16 (round to nearest even), so the same seed gives the same bytes on every
machine. Shapes follow the workloads of vLLM PR #64659 ("GEMM-RS
microbenchmark": N=6144, K=2048 for o_proj and K=3072 for down_proj, M = tokens).
"""
import torch

HIDDEN = 6144          # N of o_proj / down_proj and the norm width
K_O_PROJ = 2048        # o_proj K per rank
K_DOWN_PROJ = 3072     # down_proj K per rank


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape, sigma: float, seed: int) -> torch.Tensor:
    """BF16 tensor of N(0, sigma^2) draws (fp32 randn * sigma, rounded to BF16)."""
    g = _gen(seed)
    return (torch.randn(tuple(shape), dtype=torch.float32, generator=g) * sigma).to(torch.bfloat16)


def activations_bf16(m: int, k: int, seed: int = 0) -> torch.Tensor:
    """o_proj-style input: BF16 [m, k] ~ N(0, 1)."""
    return normal_bf16((m, k), 1.0, seed)


def gated_activations_bf16(m: int, k: int, seed: int = 0) -> torch.Tensor:
    """down_proj-style input: BF16 of silu(g) * u in fp32, g and u ~ N(0, 1) drawn in that order."""
    gen = _gen(seed)
    g = torch.randn((m, k), dtype=torch.float32, generator=gen)
    u = torch.randn((m, k), dtype=torch.float32, generator=gen)
    return (torch.nn.functional.silu(g) * u).to(torch.bfloat16)


def weights_bf16(n: int, k: int, seed: int = 1, sigma: float = 0.02) -> torch.Tensor:
    """Linear weight in nn.Linear layout: BF16 [n, k] (K contiguous) ~ N(0, sigma^2)."""
    return normal_bf16((n, k), sigma, seed)


def norm_inputs_bf16(m: int, hidden: int, seed_x: int = 2, seed_w: int = 3,
                     outlier_frac: float = 0.01, outlier_scale: float = 50.0):
    """Norm input x [m, hidden] ~ N(0,1) with a random 1% of entries multiplied by 50
    (mask drawn after x from the same generator, applied in fp32 before the BF16
    rounding), and the norm weight w [hidden] ~ N(0, 0.1^2)."""
    gen = _gen(seed_x)
    x = torch.randn((m, hidden), dtype=torch.float32, generator=gen)
    mask = torch.rand((m, hidden), generator=gen) < outlier_frac
    x = torch.where(mask, x * outlier_scale, x)
    w = normal_bf16((hidden,), 0.1, seed_w)
    return x.to(torch.bfloat16), w


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a CPU BF16 tensor's bit patterns."""
    import numpy as np
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)
