"""Seeded synthetic inputs for the WKV workloads.

This module draws random tensors and nothing else: it holds none of the
operator's arithmetic, so both the HIP path's tests and the float64 oracle can
consume its output.  Every tensor comes from its own torch generator, seeded by
``(base, workload, index, tensor_id)`` through numpy's SeedSequence, and is
drawn in float32 on the requested device.  The oracle always reads back the
exact float32 values the GPU consumed, so host and device generators never have
to agree bit for bit.

Tensor ids: 0 decay, 1 u, 2 k, 3 v, 4 dy, 5 outlier positions, 6 outlier signs,
7 receptance r (the output gate's input), 8 token-shift input x, 9 token-shift
weights mu, 10 carried last token x_prev.

The distributions follow the workloads shaped like the pages' models
(24 layers x 2048 wide, 4096 x 24, a 1M-token document in 1024-token chunks):
the per-channel decay parameter is uniform and w = exp(decay) > 0 (the pages
parametrise the decay rate that way so it is always positive); u, k, v and dy
are normal with the stated standard deviation.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

TID_DECAY, TID_U, TID_K, TID_V, TID_DY, TID_POS, TID_SIGN, TID_R, TID_X, TID_MU, TID_XPREV = \
    range(11)


def seed_of(workload: int, index: int, tensor_id: int, base: int = 0) -> int:
    ss = np.random.SeedSequence([base, workload, index, tensor_id])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _generator(device, seed: int) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev.type if dev.type != "cuda" else dev)
    g.manual_seed(seed)
    return g


def uniform(shape, lo: float, hi: float, seed: int, device="cpu") -> torch.Tensor:
    """float32 U[lo, hi) (half-open)."""
    g = _generator(device, seed)
    x = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(hi - lo).add_(lo)


def normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    """float32 N(0, std^2); the second parameter is the standard deviation."""
    g = _generator(device, seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)


@dataclass(frozen=True)
class Recipe:
    """Distribution parameters of one workload's inputs."""
    decay_lo: float = -5.0
    decay_hi: float = 1.0
    u_std: float = 0.5
    k_std: float = 1.0
    v_std: float = 1.0
    outlier_frac: float = 0.0     # fraction of k entries overwritten by +-outlier_mag
    outlier_mag: float = 60.0
    r_std: float = 2.0            # receptance: sigmoid(r) spans most of (0, 1)


# Workload ids and their recipes.
TINY = 0        # B=1 T=64 C=32
GPT = 1         # B=8 T=1024 C=2048, one layer per call, 24 layers
STREAM = 2      # B=1 C=5120, 1024 chunks of 1024 tokens with the state carried
DECODE = 3      # L=24 B=1024 C=4096, T=1 steps after 256 warm-up tokens
STABILITY = 4   # B=8 T=4096 C=2048, wide exponents, forward + backward

RECIPES = {
    TINY: Recipe(),
    GPT: Recipe(k_std=2.0),
    STREAM: Recipe(),
    DECODE: Recipe(),
    STABILITY: Recipe(decay_lo=-8.0, decay_hi=3.0, u_std=2.0, k_std=8.0,
                      outlier_frac=1e-3, outlier_mag=60.0),
}

SHAPES = {
    TINY: dict(B=1, T=64, C=32),
    GPT: dict(B=8, T=1024, C=2048, layers=24),
    STREAM: dict(B=1, T=1024, C=5120, chunks=1024),
    DECODE: dict(L=24, B=1024, C=4096, warmup=256, steps=512, ring=32),
    STABILITY: dict(B=8, T=4096, C=2048),
}


def channel_params(workload: int, index: int, C: int, device="cpu", recipe: Recipe = None):
    """Per-channel (w, u), each [C] float32, w = exp(decay)."""
    r = recipe or RECIPES[workload]
    decay = uniform((C,), r.decay_lo, r.decay_hi, seed_of(workload, index, TID_DECAY), device)
    w = torch.exp(decay)
    u = normal((C,), r.u_std, seed_of(workload, index, TID_U), device)
    return w, u


def sequence(workload: int, index: int, shape, device="cpu", recipe: Recipe = None,
             with_dy: bool = False):
    """k, v (and dy) of the given shape (e.g. [B][T][C]) as float32 tensors."""
    r = recipe or RECIPES[workload]
    k = normal(shape, r.k_std, seed_of(workload, index, TID_K), device)
    if r.outlier_frac > 0.0:
        n_total = k.numel()
        n = int(round(r.outlier_frac * n_total))
        if n > 0:
            gp = _generator(device, seed_of(workload, index, TID_POS))
            pos = torch.randperm(n_total, generator=gp, device=device)[:n]
            gs = _generator(device, seed_of(workload, index, TID_SIGN))
            sign = torch.randint(0, 2, (n,), generator=gs, device=device).to(torch.float32)
            k.view(-1)[pos] = (sign * 2.0 - 1.0) * r.outlier_mag
    v = normal(shape, r.v_std, seed_of(workload, index, TID_V), device)
    if not with_dy:
        return k, v
    dy = normal(shape, 1.0, seed_of(workload, index, TID_DY), device)
    return k, v, dy


def receptance(workload: int, index: int, shape, device="cpu", recipe: Recipe = None):
    """The gate's receptance r (before the sigmoid), float32 of the given shape."""
    r = recipe or RECIPES[workload]
    return normal(shape, r.r_std, seed_of(workload, index, TID_R), device)


def shift_inputs(workload: int, index: int, B: int, T: int, C: int, M: int, device="cpu"):
    """Token-shift inputs: mu [M][C] ~ U(0, 1) (an interpolation weight),
    x [B][T][C] ~ N(0, 1) (a layer-normalised embedding), x_prev [B][C] ~ N(0, 1)."""
    mu = uniform((M, C), 0.0, 1.0, seed_of(workload, index, TID_MU), device)
    x = normal((B, T, C), 1.0, seed_of(workload, index, TID_X), device)
    xp = normal((B, C), 1.0, seed_of(workload, index, TID_XPREV), device)
    return mu, x, xp


def make(workload: int, index: int = 0, device="cpu", B=None, T=None, C=None,
         with_dy: bool = False, recipe: Recipe = None):
    """Inputs of one forward (or forward+backward) call: dict of w, u, k, v[, dy]."""
    sh = SHAPES[workload]
    B = sh.get("B") if B is None else B
    T = sh.get("T") if T is None else T
    C = sh.get("C") if C is None else C
    w, u = channel_params(workload, index, C, device, recipe)
    seq = sequence(workload, index, (B, T, C), device, recipe, with_dy)
    out = dict(w=w, u=u, k=seq[0], v=seq[1])
    if with_dy:
        out["dy"] = seq[2]
    return out
