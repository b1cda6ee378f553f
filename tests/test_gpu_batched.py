"""GPU parity of grouped launches at a decode batch, 2 <= M <= 16 (needs gfx950).

The kernel decodes each packed byte once and runs the M-token products on the
matrix cores; products of codes and bf16 activations are exact and sums are
fp32, so the GEMV bar applies: max_n |dy| / ||y_row||_2 <= 2e-3 against the
oracle (fp64), with a normwise tripwire far below it.  Shapes cover ragged row
counts, every grid and mixed row blocks, and row lengths whose ternary tail
ends inside a chunk (K = 128, 384, 512, 1280, 5120) or a period.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2
TOL, TRIP = 2e-3, 1e-5

CASES = [(1, 128, T), (3, 256, I2), (64, 640, I3), (129, 1280, "mixed"), (70, 384, T), (200, 512, T),
         (1000, 4096, "mixed"), (130, 5120, T), (256, 12288, "mixed"), (65, 2048, I3), (300, 4096, I2),
         (97, 384, I3), (64, 128, I2)]


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def grid_arg(N, grid, seed):
    if grid != "mixed":
        return grid
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    t = rng.integers(0, 3, nb).astype(np.int8)
    t[: min(3, nb)] = [2, 0, 1][: min(3, nb)]
    return t


def case(ora, dev, N, K, grid, M, seed):
    g = grid_arg(N, grid, seed)
    W = synth.weight(N, K, seed=seed)
    c_ref, s_ref = ora.quantize(W.numpy(), g)
    x = synth.activations(M, K, seed=seed + 1)
    y64 = ora.gemv(c_ref, s_ref, synth.bf16_bits(x))
    return ql.quantize_pack(W.to(dev), g), x.to(dev), y64


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8, 13, 16])
def test_batched_grouped_parity(ora, dev, M):
    note(f"batched grouped M={M}")
    items, refs = [], []
    for i, (N, K, grid) in enumerate(CASES):
        pw, x, y64 = case(ora, dev, N, K, grid, M, seed=3000 + 17 * i + M)
        items.append((pw, x, torch.full((M, N), float("nan"), device=dev)))
        refs.append(y64)
    grp = ql.GroupedGemv(items)
    grp.run()
    torch.cuda.synchronize()
    for (pw, x, y), y64 in zip(items, refs):
        err, normwise = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= TOL and normwise <= TRIP, (pw.N, pw.K, pw.grid, M, err, normwise)
    # the scheduler state is left zero and a repeated launch is bitwise identical
    assert int(grp.sched.abs().sum().item()) == 0
    first = [y.clone() for _, _, y in items]
    grp.run()
    torch.cuda.synchronize()
    assert int(grp.sched.abs().sum().item()) == 0
    for (_, _, y), y1 in zip(items, first):
        assert torch.equal(y, y1)


def test_batched_matches_batch1_rows(ora, dev):
    """Each token row of a batched launch agrees with a batch-1 launch of that row (both
    within the bar of the exact result; their MFMA sums of the other token groups differ)."""
    note("batched vs batch-1 rows")
    N, K, M = 384, 4096, 6
    g = grid_arg(N, "mixed", 77)
    W = synth.weight(N, K, seed=77, device=dev)
    pw = ql.quantize_pack(W, g)
    x = synth.activations(M, K, seed=78, device=dev)
    y = torch.empty((M, N), device=dev)
    ql.GroupedGemv([(pw, x, y)]).run()
    for m in range(M):
        y1 = torch.empty((1, N), device=dev)
        ql.GroupedGemv([(pw, x[m:m + 1].contiguous(), y1)]).run()
        torch.cuda.synchronize()
        d = (y[m] - y1[0]).abs().max().item() / max(y1[0].norm().item(), 1e-30)
        assert d <= 1e-5, (m, d)


def test_batched_rejects_m_above_16(dev):
    N, K = 64, 256
    pw = ql.quantize_pack(synth.weight(N, K, seed=5, device=dev), T)
    x = synth.activations(17, K, seed=6, device=dev)
    grp = ql.GroupedGemv([(pw, x, torch.empty((17, N), device=dev))])
    with pytest.raises(ql.QLinearError):
        grp.run()
