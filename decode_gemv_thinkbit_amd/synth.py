"""Seeded synthetic inputs shared by the oracle tests and the GPU path.

This module draws random numbers and lays out grid allocations; it holds
none of the quantization or product arithmetic.  Both sides of every parity
check receive exactly the arrays it returns.

* Weights: W ~ N(0, 0.02^2) in fp32 (``torch.randn`` with a seeded
  generator, times 0.02).  The trained Qwen3 ThinkBit checkpoints that the
  summary page serves are not available; these stand in for them with the
  same shapes.
* Activations: x ~ N(0, 1), rounded to bf16 by torch.
* LittleBit parameters (``littlebit_params``): random signs and log-normal
  scales of the page's shapes.
* Output gradients for the allocator's sensitivities: N(0, sigma^2) with a
  log-normal sigma per linear (``output_gradient``).
* Mixed allocation (summary page onedev.kr/papers/1416, section "How it
  differs": 75.3 % ternary, 6.0 % 2-bit, 18.7 % 3-bit of a layer's weights;
  query/key kept at >= 2 bits, here forced to 3 bits): per layer, every
  128-row block of the forced linears is 3-bit; the remaining blocks are
  shuffled with a seeded permutation and assigned 3-bit until the layer's
  3-bit share reaches 18.7 %, then 2-bit until 6.0 %, the rest ternary.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import (BASE_SEED, GRID_I2, GRID_I3, GRID_MIXED, GRID_T, SHARE_I2, SHARE_I3, W_SIGMA,
                      Workload)

BLOCK_ROWS = 128


def seed_of(*parts: int) -> int:
    """A 63-bit seed derived from integer parts (numpy SeedSequence)."""
    ss = np.random.SeedSequence([BASE_SEED] + [int(p) for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0] >> np.uint64(1))


def weight(N: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(N, K, generator=g, device=device, dtype=torch.float32) * W_SIGMA


def activations(M: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    """bf16 tensor [M][K]."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(M, K, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def n_blocks(N: int) -> int:
    return (N + BLOCK_ROWS - 1) // BLOCK_ROWS


def layer_allocation(linears, seed: int, forced_i3=("q", "k")) -> dict:
    """Grid of every 128-row block of every linear of one layer -> {name: int8 array}."""
    out = {l.name: np.full(n_blocks(l.N), GRID_T, dtype=np.int8) for l in linears}
    total = sum(l.N * l.K for l in linears)
    i3 = 0
    free = []
    for li, l in enumerate(linears):
        for b in range(n_blocks(l.N)):
            w = (min(BLOCK_ROWS, l.N - b * BLOCK_ROWS)) * l.K
            if l.name in forced_i3:
                out[l.name][b] = GRID_I3
                i3 += w
            else:
                free.append((li, b, w))
    order = np.random.default_rng(seed).permutation(len(free))
    i2 = 0
    for idx in order:
        li, b, w = free[idx]
        name = linears[li].name
        if i3 < SHARE_I3 * total:
            out[name][b] = GRID_I3
            i3 += w
        elif i2 < SHARE_I2 * total:
            out[name][b] = GRID_I2
            i2 += w
    return out


def allocation(wl: Workload, layer: int) -> dict:
    if wl.grid != GRID_MIXED:
        return {l.name: np.full(n_blocks(l.N), wl.grid, dtype=np.int8) for l in wl.linears}
    return layer_allocation(list(wl.linears), seed_of(7, layer, len(wl.linears), wl.layers), wl.forced_i3)


def realized_shares(wl: Workload) -> dict:
    """Fraction of the workload's weights on each grid."""
    tot = {GRID_T: 0, GRID_I2: 0, GRID_I3: 0}
    for layer in range(wl.layers):
        alloc = allocation(wl, layer)
        for l in wl.linears:
            for b, g in enumerate(alloc[l.name]):
                tot[int(g)] += min(BLOCK_ROWS, l.N - b * BLOCK_ROWS) * l.K
    s = sum(tot.values())
    return {k: v / s for k, v in tot.items()}


def output_gradient(N: int, wl_index: int, layer: int, mat: int, device="cpu") -> torch.Tensor:
    """Synthetic output gradient of one linear, fp32 [N]: N(0, sigma^2) per element with a
    per-linear log-normal sigma = exp(z / 2), z ~ N(0, 1).  (The real gradients come from
    calibration data on a trained model, which this build does not have.)"""
    rng = np.random.default_rng(seed_of(5, wl_index, layer, mat))
    sigma = float(np.exp(0.5 * rng.standard_normal()))
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(6, wl_index, layer, mat))
    return torch.randn(N, generator=g, device=device, dtype=torch.float32) * sigma


def littlebit_params(d_out: int, d_in: int, r: int, seed: int, device="cpu"):
    """Seeded parameters of a two-path LittleBit linear: signs +-1 with probability 1/2
    (int8 [2, d_out, r] and [2, d_in, r]); bf16 scales g = exp(0.25 z) [2, d_in],
    l = exp(0.5 z) / sqrt(r) [2, r], h = 0.02 exp(0.25 z) [2, d_out], z ~ N(0, 1).
    (Trained LittleBit checkpoints are not available; kernel time does not depend on the
    values.)"""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def signs(*shape):
        return (torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int8) * 2 - 1).to(torch.int8)

    u = signs(2, d_out, r)
    v = signs(2, d_in, r)
    g = torch.exp(0.25 * torch.randn(2, d_in, generator=gen, device=device)).to(torch.bfloat16)
    l = (torch.exp(0.5 * torch.randn(2, r, generator=gen, device=device)) / float(np.sqrt(r))).to(torch.bfloat16)
    h = (0.02 * torch.exp(0.25 * torch.randn(2, d_out, generator=gen, device=device))).to(torch.bfloat16)
    return u, v, g, l, h


def weight_seed(wl_index: int, layer: int, mat: int) -> int:
    return seed_of(1, wl_index, layer, mat)


def x_seed(wl_index: int, layer: int, slot: str, M: int) -> int:
    return seed_of(2, wl_index, layer, {"attn": 0, "o": 1, "mlp": 2, "down": 3}[slot], M)
