"""Grid allocation of a workload by the Lagrangian multiple-choice knapsack.

ThinkBit summary page (onedev.kr/papers/1416), section "How it differs",
stage 1 (Allocate): the sensitivity of a layer is the product of the squared
norms of its input activations and of its output gradients; times the
rounding noise of a grid it approximates the loss increase of that grid; one
grid per unit is chosen under a bit budget for the whole decoder by
Lagrangian relaxation, with query and key projections kept at >= 2 bits.

The rounding noise and the sensitivities run on the GPU
(``qlinear_rtn_noise``, ``qlinear_block_sensitivity``), the knapsack in the
library's host code (``qlinear_allocate``); this module only gathers the
units.  A unit is a 128-row grid block (the granularity the packed layout
stores) or a whole linear.  The activations are the workload's own seeded
x; the output gradients are seeded stand-ins (``synth.output_gradient``).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import qlinear as ql
from . import synth
from .configs import Workload

BLOCK_ROWS = 128


@dataclass
class Units:
    keys: list            # (layer, linear name, first block, blocks) per unit
    weights: np.ndarray   # int64
    sensitivity: np.ndarray
    noise: np.ndarray     # [units][3]
    allowed: np.ndarray   # uint32 masks


def workload_units(wl: Workload, wl_index: int, dev, layers=None, granularity: str = "block",
                   keep_2bit=("q", "k")) -> Units:
    """Units of the workload's decoder layers with their weights, sensitivity and noise."""
    keys, n, S, E, allowed = [], [], [], [], []
    for layer in (range(wl.layers) if layers is None else layers):
        for mi, lin in enumerate(wl.linears):
            W = synth.weight(lin.N, lin.K, synth.weight_seed(wl_index, layer, mi), device=dev)
            noise = ql.rtn_noise(W).cpu().numpy()
            del W
            x = synth.activations(1, lin.K, synth.x_seed(wl_index, layer, lin.x_slot, 1), device=dev)
            sb = ql.block_sensitivity(x, synth.output_gradient(lin.N, wl_index, layer, mi, device=dev)).cpu().numpy()
            rows = np.minimum(BLOCK_ROWS, lin.N - BLOCK_ROWS * np.arange(len(sb)))
            mask = ql.AT_LEAST_2BIT if lin.name in keep_2bit else ql.ALL_GRIDS
            if granularity == "block":
                for b in range(len(sb)):
                    keys.append((layer, lin.name, b, 1))
                    n.append(int(rows[b]) * lin.K)
                    S.append(sb[b])
                    E.append(noise[b])
                    allowed.append(mask)
            else:  # one unit per linear: its sensitivity and noise are the blocks' sums
                keys.append((layer, lin.name, 0, len(sb)))
                n.append(lin.N * lin.K)
                S.append(float(sb.sum()))
                E.append(noise.sum(axis=0))
                allowed.append(mask)
    return Units(keys, np.asarray(n, np.int64), np.asarray(S, np.float64), np.asarray(E, np.float64).reshape(-1, 3),
                 np.asarray(allowed, np.uint32))


def tables_from(units: Units, grids: np.ndarray, wl: Workload) -> dict:
    """{layer: {linear name: int8 grid per 128-row block}} from per-unit grids."""
    out: dict = {}
    nblk = {l.name: (l.N + BLOCK_ROWS - 1) // BLOCK_ROWS for l in wl.linears}
    for (layer, name, b0, nb), g in zip(units.keys, grids):
        t = out.setdefault(layer, {}).setdefault(name, np.zeros(nblk[name], np.int8))
        t[b0:b0 + nb] = g
    return out


def knapsack_allocation(wl: Workload, wl_index: int, dev, budget_bits: float = 2.0, layers=None,
                        granularity: str = "block", grid_bits=None):
    """Grid tables for the workload's layers, and (units, grids, multiplier)."""
    units = workload_units(wl, wl_index, dev, layers, granularity)
    grids, lam = ql.allocate(units.weights, units.sensitivity, units.noise, units.allowed, budget_bits, grid_bits)
    return tables_from(units, grids, wl), (units, grids, lam)


def shares(units: Units, grids: np.ndarray) -> dict:
    tot = units.weights.sum()
    return {g: float(units.weights[grids == g].sum() / tot) for g in range(3)}
