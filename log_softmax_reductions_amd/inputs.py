"""Seeded synthetic inputs for the five workloads (and for tests of any shape).

This module draws random numbers and nothing else: it holds none of the
reduction arithmetic, so both the HIP path and the fp64 oracle can be fed from
it without sharing any of the method's code.  Every draw goes through a
``torch.Generator`` seeded explicitly, on the device the data is wanted on
(Philox on the GPU, Mersenne Twister on the CPU); the same seed on the same
device kind gives the same bytes.  Data made on the GPU is copied to the host
before the oracle sees it, so the oracle always gets the exact fp32 values the
kernels read.

Workloads (shapes and distributions as the three pages state them):
  axis0_small  logsumexp over dim 0 of (4, 10, 32), N(0, 1)
  rows_small   log_softmax over dim 1 of (128, 4096), N(0, 1); 1% of entries
               scaled by 50, then 1% set to -inf (two independent masks, the
               -inf mask applied last); no row is left entirely -inf
  axis0_large  logsumexp over dim 0 of (32, 2048, 4096), N(0, variance 4)
  rows_large   log_softmax over dim 1 of (4096, 393216), N(0, 1)
  conv_chain   x (128, 8, 128, 128) N(0, 1); conv weight and bias
               U(-1/sqrt(72), 1/sqrt(72)) (PyTorch's default Conv2d bound for
               fan-in 8*3*3); GroupNorm gamma = 1, beta = 0
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

WORKLOAD_SEEDS = {
    "axis0_small": 1,
    "rows_small": 2,
    "axis0_large": 3,
    "rows_large": 4,
    "conv_chain": 5,
}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "axis0" | "rows" | "conv_chain"
    shape: tuple
    seed: int
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "axis0_small": Workload("axis0_small", "axis0", (4, 10, 32), 1, {"sigma": 1.0}),
    "rows_small": Workload("rows_small", "rows", (128, 4096), 2,
                           {"scale_frac": 0.01, "scale": 50.0, "ninf_frac": 0.01}),
    "axis0_large": Workload("axis0_large", "axis0", (32, 2048, 4096), 3, {"sigma": 2.0}),
    "rows_large": Workload("rows_large", "rows", (4096, 393216), 4, {}),
    "conv_chain": Workload("conv_chain", "conv_chain", (128, 8, 128, 128), 5,
                           {"cout": 64, "k": 3, "groups": 16, "eps": 1e-5}),
}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, sigma: float = 1.0, device="cpu",
           gen: torch.Generator | None = None) -> torch.Tensor:
    """i.i.d. N(0, sigma^2) fp32 of the given shape."""
    g = gen if gen is not None else generator(seed, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x


def uniform(shape, bound: float, device="cpu", gen: torch.Generator = None) -> torch.Tensor:
    """i.i.d. U(-bound, bound) fp32."""
    u = torch.rand(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    return u.mul_(2.0 * bound).sub_(bound)


def rows_with_outliers(rows: int, cols: int, seed: int, device="cpu",
                       scale_frac: float = 0.01, scale: float = 50.0,
                       ninf_frac: float = 0.01) -> torch.Tensor:
    """N(0,1) rows; a Bernoulli(scale_frac) mask multiplies entries by `scale`,
    then an independent Bernoulli(ninf_frac) mask sets entries to -inf.  A row
    the -inf mask would empty keeps its first entry finite."""
    g = generator(seed, device)
    x = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
    if scale_frac > 0:
        m = torch.rand((rows, cols), generator=g, device=device) < scale_frac
        x = torch.where(m, x * scale, x)
    if ninf_frac > 0:
        m = torch.rand((rows, cols), generator=g, device=device) < ninf_frac
        x = x.masked_fill(m, float("-inf"))
        full = torch.isneginf(x).all(dim=1)
        if bool(full.any()):
            x[full, 0] = 0.0
    return x.contiguous()


def conv_chain_inputs(N=128, Cin=8, H=128, W=128, Cout=64, K=3, seed=5, device="cpu"):
    """(x, weight, bias, gamma, beta) for the conv -> GroupNorm -> ... chain."""
    g = generator(seed, device)
    x = torch.randn((N, Cin, H, W), generator=g, device=device, dtype=torch.float32)
    bound = 1.0 / math.sqrt(Cin * K * K)
    w = uniform((Cout, Cin, K, K), bound, device, g)
    b = uniform((Cout,), bound, device, g)
    gamma = torch.ones(Cout, device=device, dtype=torch.float32)
    beta = torch.zeros(Cout, device=device, dtype=torch.float32)
    return x, w, b, gamma, beta


def make(name: str, device="cpu"):
    """Inputs of a named workload: a tensor, or the chain's 5-tuple."""
    wl = WORKLOADS[name]
    if wl.kind == "axis0":
        return normal(wl.shape, wl.seed, wl.params.get("sigma", 1.0), device)
    if wl.kind == "rows":
        rows, cols = wl.shape
        p = wl.params
        if p:
            return rows_with_outliers(rows, cols, wl.seed, device, p["scale_frac"],
                                      p["scale"], p["ninf_frac"])
        return normal(wl.shape, wl.seed, 1.0, device)
    N, Cin, H, W = wl.shape
    return conv_chain_inputs(N, Cin, H, W, wl.params["cout"], wl.params["k"],
                             wl.seed, device)
