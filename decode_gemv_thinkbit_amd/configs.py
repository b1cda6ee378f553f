"""The synthetic workloads, as data only (shapes, grids, batch sizes).

Shapes follow the Qwen3 decoder layers that the ThinkBit summary page
(onedev.kr/papers/1416), section "Premises & limits", serves at batch 1
(1.7B, 8B and 14B models).  The allocation fractions 75.3 % ternary /
6.0 % 2-bit / 18.7 % 3-bit come from the same page, section "How it
differs" (Qwen3-1.7B at a 2.0-bit budget).  Weights are synthetic:
W ~ N(0, 0.02^2) in fp32 and x ~ N(0, 1) rounded to bf16, both seeded.
"""
from __future__ import annotations

from dataclasses import dataclass

GRID_T, GRID_I2, GRID_I3, GRID_MIXED = 0, 1, 2, 3
GRID_NAMES = {GRID_T: "T", GRID_I2: "I2", GRID_I3: "I3", GRID_MIXED: "mixed"}

# Allocation shares by weight (summary page, section "How it differs").
SHARE_T, SHARE_I2, SHARE_I3 = 0.753, 0.060, 0.187

W_SIGMA = 0.02
BASE_SEED = 1416


@dataclass(frozen=True)
class Linear:
    name: str
    N: int  # output rows
    K: int  # input columns
    x_slot: str  # which activation feeds it within a layer


def qwen3_layer(hidden: int, kv: int, inter: int) -> list[Linear]:
    """The seven linears of one decoder layer; q/k/v share x_attn, gate/up share x_mlp."""
    return [
        Linear("q", hidden, hidden, "attn"),
        Linear("k", kv, hidden, "attn"),
        Linear("v", kv, hidden, "attn"),
        Linear("o", hidden, hidden, "o"),
        Linear("gate", inter, hidden, "mlp"),
        Linear("up", inter, hidden, "mlp"),
        Linear("down", hidden, inter, "down"),
    ]


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    linears: tuple
    grid: int  # a uniform grid, or GRID_MIXED
    M: tuple = (1,)
    forced_i3: tuple = ()  # linears forced to 3-bit in a mixed allocation

    @property
    def weights(self) -> int:
        return self.layers * sum(l.N * l.K for l in self.linears)


LAYER_1P7B = tuple(qwen3_layer(2048, 1024, 6144))
LAYER_8B = tuple(qwen3_layer(4096, 1024, 12288))
LAYER_14B = tuple(qwen3_layer(5120, 1024, 17408))

WORKLOADS = {
    # one 2048x2048 linear, uniform 2-bit grid, batch 1
    "linear2048_i2": Workload("linear2048_i2", 1, (Linear("w", 2048, 2048, "attn"),), GRID_I2),
    # one Qwen3-1.7B-shaped decoder layer, mixed grids, q and k at 3 bits
    "qwen3_1p7b_layer": Workload("qwen3_1p7b_layer", 1, LAYER_1P7B, GRID_MIXED, forced_i3=("q", "k")),
    # the linears of one Qwen3-8B decode step: 36 layers, mixed grids
    "qwen3_8b_pass": Workload("qwen3_8b_pass", 36, LAYER_8B, GRID_MIXED, forced_i3=("q", "k")),
    # Qwen3-14B-shaped stack: 40 layers, mixed grids, batch 1/4/16
    "qwen3_14b_stack": Workload("qwen3_14b_stack", 40, LAYER_14B, GRID_MIXED, M=(1, 4, 16),
                                forced_i3=("q", "k")),
    # Qwen3-8B layer shapes at prefill/batched-decode sizes, each grid separately and mixed
    "qwen3_8b_gemm": Workload("qwen3_8b_gemm", 1, LAYER_8B, GRID_MIXED, M=(64, 256, 512), forced_i3=("q", "k")),
}
