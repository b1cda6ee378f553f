"""One-hot probes of the decode kernels that the benchmark times (needs gfx950).

x = e_k gives y[n] = c[n,k] * s[n,k/128] exactly: one exact product, the rest
zeros, and an exact scale multiply (c * s needs at most 10 significant bits).
So every position's decode is checked bit for bit, not through a tolerance.
This is the GPU pin of the ThinkBit summary page (onedev.kr/papers/1416),
section "How it works": dequantization is one multiply.

Positions: every residue mod 80 (ternary chunk), mod 16 (2-bit word) and
mod 32 (3-bit triple), both ends of the row, a 640-input period edge, the
first and last 128-input group, and the ternary padding edge (K % 80 != 0).

Paths:
  * qlinear_gemv at M = 1, one launch per position (gemv_kernel<1>);
  * the grouped batch-1 launch (gemv_grouped_kernel<1>), every item a
    different position against the same weight, with and without split-K;
  * the grouped batched-decode launch at M = 4 and 16
    (gemv_grouped_kernel, one and four token groups), token t of an item
    holding its own position.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def mixed_table(N, seed):
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    t = rng.integers(0, 3, nb).astype(np.int8)
    t[: min(3, nb)] = [0, 2, 1][: min(3, nb)]
    return t


def positions(K):
    """Every residue mod 80 / 16 / 32 near the start, a period edge, the last group and the tail."""
    ks = set(range(0, min(K, 160)))
    ks |= set(range(max(0, 630), min(K, 660)))
    ks |= set(range(max(0, K - 130), K))
    return sorted(ks)


def weight_case(ora, dev, N, K, grid, seed):
    g = mixed_table(N, seed) if grid == "mixed" else grid
    W = synth.weight(N, K, seed=seed)
    c_ref, s_ref = ora.quantize(W.numpy(), g)
    w32, _ = ora.dequant(c_ref, s_ref)
    pw = ql.quantize_pack(W.to(dev), g)
    return pw, w32


def one_hot(ks, K, dev):
    X = torch.zeros((len(ks), K), dtype=torch.bfloat16)
    X[torch.arange(len(ks)), torch.tensor(ks)] = 1.0
    return X.to(dev)


def assert_columns(Y, w32, ks, what):
    for i, k in enumerate(ks):
        if not np.array_equal(Y[i], w32[:, k]):
            bad = np.flatnonzero(Y[i] != w32[:, k])
            raise AssertionError(f"{what}: k={k}: rows {bad[:8].tolist()} got {Y[i][bad[:4]].tolist()} "
                                 f"want {w32[bad[:4], k].tolist()}")


# (N, K): K = 1280 ends on a chunk edge; 4096 and 384 end inside a ternary chunk
# (the padding edge); 5120 spans several 640-input periods exactly.
SHAPES = [(130, 1280), (64, 4096), (70, 384), (129, 5120)]
GRIDS = [T, I2, I3, "mixed"]


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", GRIDS)
def test_gemv_batch1_one_hot(ora, dev, N, K, grid):
    """qlinear_gemv at M = 1 (the single-matrix form of the decode GEMV), one launch per position."""
    note(f"one-hot gemv M=1 N={N} K={K} grid={grid}")
    pw, w32 = weight_case(ora, dev, N, K, grid, seed=11 * N + K)
    ks = positions(K)
    X = one_hot(ks, K, dev)
    # one output tensor per launch: the library takes 16-byte aligned pointers only
    Y = [torch.full((1, N), float("nan"), device=dev) for _ in ks]
    for i in range(len(ks)):
        ql.gemv(X[i:i + 1], pw, out=Y[i])
    assert_columns(torch.cat(Y).cpu().numpy(), w32, ks, "gemv M=1")


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("split", [None, 3, "auto"])
def test_grouped_batch1_one_hot(ora, dev, N, K, grid, split):
    """The grouped batch-1 launch: one item per position, all against one weight; split-K
    parts (forced 3, or automatic) must leave every value exact too."""
    note(f"one-hot grouped M=1 N={N} K={K} grid={grid} split={split}")
    pw, w32 = weight_case(ora, dev, N, K, grid, seed=13 * N + K)
    ks = positions(K)
    X = one_hot(ks, K, dev)
    Y = [torch.full((1, N), float("nan"), device=dev) for _ in ks]
    items = [(pw, X[i:i + 1], Y[i]) for i in range(len(ks))]
    grp = ql.GroupedGemv(items, split=split)
    for rep in range(2):
        grp.run()
        torch.cuda.synchronize()
        assert int(grp.sched.abs().sum().item()) == 0 or split is not None
        assert_columns(torch.cat(Y).cpu().numpy(), w32, ks, f"grouped M=1 split={split} rep {rep}")
        for y in Y:
            y.fill_(float("nan"))


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("M", [4, 16])
def test_grouped_batched_one_hot(ora, dev, N, K, grid, M):
    """The grouped launch at M = 4 and 16: token t of item i probes position ks[i*M + t]."""
    note(f"one-hot batched M={M} N={N} K={K} grid={grid}")
    pw, w32 = weight_case(ora, dev, N, K, grid, seed=17 * N + K + M)
    ks = positions(K)
    ks = ks + ks[: (-len(ks)) % M]  # whole items of M tokens
    X = one_hot(ks, K, dev)
    Y = [torch.full((M, N), float("nan"), device=dev) for _ in range(0, len(ks), M)]
    items = [(pw, X[i:i + M], Y[i // M]) for i in range(0, len(ks), M)]
    for split in (None, "auto"):
        ql.GroupedGemv(items, split=split).run()
        torch.cuda.synchronize()
        assert_columns(torch.cat(Y).cpu().numpy(), w32, ks, f"batched M={M} split={split}")
        for y in Y:
            y.fill_(float("nan"))
