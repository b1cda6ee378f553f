"""GPU parity of split-K grouped launches (needs gfx950).

Each slab's input is cut into parts of whole 640-input periods, each part a
task; the wave that finishes a slab's last part sums the parts' fp32 partial
sums in part order.  The bar is the GEMV's: max_n |dy| / ||y_row||_2 <= 2e-3
against the oracle (fp64), normwise tripwire 1e-5, at batch 1 and at batches of
four and sixteen tokens.  Shapes cover one-period rows (no split possible),
ternary tails inside a chunk or period, every grid and mixed blocks, parts that
do not divide the periods, and as many parts as periods.  Repeat launches are
bitwise identical and leave every counter at zero.
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

# (N, K, grid): periods per row 1, 2, 7, 8, 20, 3, 7, 7
CASES = [(64, 128, T), (130, 1280, I2), (200, 4096, "mixed"), (97, 5120, T), (128, 12288, I3), (65, 1920, T),
         (300, 4096, I2), (70, 4096, T)]


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


def build(ora, dev, M, seed0):
    items, refs = [], []
    for i, (N, K, grid) in enumerate(CASES):
        seed = seed0 + 31 * i
        g = grid_arg(N, grid, seed)
        W = synth.weight(N, K, seed=seed)
        c_ref, s_ref = ora.quantize(W.numpy(), g)
        x = synth.activations(M, K, seed=seed + 1)
        refs.append(ora.gemv(c_ref, s_ref, synth.bf16_bits(x)))
        items.append((ql.quantize_pack(W.to(dev), g), x.to(dev), torch.full((M, N), float("nan"), device=dev)))
    return items, refs


def counters_zero(grp):
    """Every queue word and every split counter line of the launch's state is zero."""
    st = grp.sched.cpu().numpy()
    ok = not st[: ql.QL_SCHED_WORDS].any()
    for d in grp.plan:
        if d["kparts"] > 1:
            ns = (d["N"] + 63) // 64
            ok = ok and not st[d["ws_begin"]: d["ws_begin"] + 32 * ns].any()
    return ok


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("split", [2, 3, 7, 64, "auto"])
def test_split_grouped_parity(ora, dev, M, split):
    note(f"split grouped M={M} split={split}")
    items, refs = build(ora, dev, M, seed0=5000 + 7 * M)
    grp = ql.GroupedGemv(items, split=split)
    assert max(grp.kparts) > 1
    grp.run()
    torch.cuda.synchronize()
    for (pw, x, y), y64 in zip(items, refs):
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= TOL and nw <= TRIP, (pw.N, pw.K, pw.grid, M, split, err, nw)
    assert counters_zero(grp)
    first = [y.clone() for _, _, y in items]
    for _, _, y in items:
        y.fill_(float("nan"))
    grp.run()
    torch.cuda.synchronize()
    assert counters_zero(grp)
    for (_, _, y), y1 in zip(items, first):
        assert torch.equal(y, y1)


def test_split_per_item_parts_and_unsplit_agree(ora, dev):
    """Per-item parts (one entry unsplit, one forced, one chosen) in one launch; each
    matches the unsplit launch within the sum-order bound."""
    note("split per-item parts")
    items, refs = build(ora, dev, 1, seed0=6100)
    parts = [1, 5, 0, 2, 20, 0, 7, 3]
    grp = ql.GroupedGemv(items, split=parts)
    grp.run()
    torch.cuda.synchronize()
    split_y = [y.clone() for _, _, y in items]
    ql.GroupedGemv(items).run()
    torch.cuda.synchronize()
    for (pw, _, y), ys, y64 in zip(items, split_y, refs):
        err, nw = ora.rel_err(ys.cpu().numpy(), y64)
        assert err <= TOL and nw <= TRIP, (pw.N, pw.K, err, nw)
        d = (ys - y).abs().max().item() / max(y.norm().item(), 1e-30)
        assert d <= 1e-5, (pw.N, pw.K, d)


@pytest.mark.parametrize("M", [1, 4])
def test_split_partials_never_stale(ora, dev, M):
    """A second launch on new activations (same state buffer) meets the oracle of the new
    activations: no part reads partial sums left by the previous launch."""
    note(f"split fresh partials M={M}")
    items, _ = build(ora, dev, M, seed0=7300 + M)
    grp = ql.GroupedGemv(items, split="auto")
    grp.run()
    torch.cuda.synchronize()
    refs = []
    for i, ((pw, x, y), (N, K, grid)) in enumerate(zip(items, CASES)):
        seed = 7300 + M + 31 * i
        W = synth.weight(N, K, seed=seed)
        c_ref, s_ref = ora.quantize(W.numpy(), grid_arg(N, grid, seed))
        x2 = synth.activations(M, K, seed=seed + 999)
        refs.append(ora.gemv(c_ref, s_ref, synth.bf16_bits(x2)))
        x.copy_(x2.to(dev))
        y.fill_(float("nan"))
    grp.run()
    torch.cuda.synchronize()
    assert counters_zero(grp)
    for (pw, _, y), y64 in zip(items, refs):
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= TOL and nw <= TRIP, (pw.N, pw.K, M, err, nw)
