"""GPU parity of the grouped GEMM (qlinear_gemm_grouped, needs gfx950).

One persistent launch of the large-tile kernel over several matrices at one M,
with the K splits the host plan chooses, then one reduction launch.  Same bar as
qlinear_gemm from 16 tokens on: max_n |dy| / ||y_row||_2 <= 1e-2 against the
oracle's fp64 product, and the oracle's product with bf16 RNE(c*s) weights
matched to fp32 summation error (normwise 1e-5); x = e_k returns RNE(c*s)
exactly; repeats are bitwise identical.  A matrix of fewer than 64 rows is held
to the bf16-weight product only: the 1e-2 bar divides by the norm of a token's
N outputs, and with three outputs the rounding of 3-bit codes of magnitude 3
(RNE(3s), the one inexact operand) can exceed it by itself.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2
GEMM_TOL, TRIP16 = 1e-2, 1e-5
# ragged row tiles, long rows (split), a 3-row matrix, every grid and mixed blocks
CASES = [(256, 4096, "mixed"), (1024, 4096, I3), (300, 12288, T), (70, 384, I2), (1000, 2048, T),
         (129, 1280, "mixed"), (520, 1920, I2), (3, 640, I3)]


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def grid_arg(N, grid, seed):
    if grid != "mixed":
        return grid
    rng = np.random.default_rng(seed)
    t = rng.integers(0, 3, (N + 127) // 128).astype(np.int8)
    t[: min(3, t.size)] = [2, 0, 1][: min(3, t.size)]
    return t


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def build(ora, dev, M, seed0):
    items, refs = [], []
    for i, (N, K, grid) in enumerate(CASES):
        seed = seed0 + 17 * i
        g = grid_arg(N, grid, seed)
        W = synth.weight(N, K, seed=seed)
        c_ref, s_ref = ora.quantize(W.numpy(), g)
        x = synth.activations(M, K, seed=seed + 1)
        y = torch.full((M, N), float("nan"), device=dev)
        items.append((ql.quantize_pack(W.to(dev), g), x.to(dev), y))
        refs.append((c_ref, s_ref, synth.bf16_bits(x)))
    return items, refs


@pytest.mark.parametrize("M", [16, 37, 64, 100, 256, 300])
def test_grouped_gemm_parity(ora, dev, M):
    note(f"grouped gemm M={M}")
    items, refs = build(ora, dev, M, seed0=900 + M)
    grp = ql.GroupedGemm(items)
    note(f"  plan {[(p['N'], p['K'], p['splits']) for p in grp.plan]} tasks {grp.total}")
    grp.run()
    torch.cuda.synchronize()
    first = [y.clone() for _, _, y in items]
    for (pw, _, y), (c_ref, s_ref, xb) in zip(items, refs):
        yy = y.cpu().numpy()
        err, normwise = ora.rel_err(yy, ora.gemv(c_ref, s_ref, xb))
        assert pw.N < 64 or err <= GEMM_TOL, (pw.N, pw.K, err, normwise)
        _, nw16 = ora.rel_err(yy, ora.gemv_w16(c_ref, s_ref, xb))
        assert nw16 <= TRIP16, (pw.N, pw.K, nw16)
    for _, _, y in items:
        y.fill_(float("nan"))
    grp.run()
    torch.cuda.synchronize()
    for (_, _, y), y0 in zip(items, first):
        assert torch.equal(y, y0)


def test_grouped_gemm_splits_long_rows(dev):
    """The plan splits K where that shortens the launch: at 512 tokens a 12288-input matrix among
    4096-input ones is cut, and every entry's tasks follow the previous entry's."""
    items = []
    for N, K in ((4096, 4096), (1024, 4096), (4096, 12288)):
        pw = ql.quantize_pack(synth.weight(N, K, seed=N + K, device=dev), T)
        items.append((pw, torch.zeros((512, K), dtype=torch.bfloat16, device=dev),
                      torch.empty((512, N), device=dev)))
    grp = ql.GroupedGemm(items)
    by_k = {p["K"]: p for p in grp.plan}
    assert by_k[12288]["splits"] > 1 and grp.ws_bytes > 0
    first = 0
    for p in grp.plan:
        assert p["first_task"] == first
        first += ((p["N"] + 255) // 256) * 2 * p["splits"]
    assert first == grp.total


@pytest.mark.parametrize("M", [16, 100])
def test_grouped_gemm_one_hot(ora, dev, M):
    """x rows = e_k: every entry returns bf16 RNE(c*s) of its weights exactly, split or not."""
    note(f"grouped gemm one-hot M={M}")
    cases = [(300, 1280, "mixed"), (256, 4096, I3), (130, 12288, T)]
    items, w16s, sels = [], [], []
    for i, (N, K, grid) in enumerate(cases):
        g = grid_arg(N, grid, 40 + i)
        W = synth.weight(N, K, seed=41 * N + K)
        c_ref, s_ref = ora.quantize(W.numpy(), g)
        _, w16 = ora.dequant(c_ref, s_ref)
        w16s.append((w16.astype(np.uint32) << 16).view(np.float32))
        sel = sorted(set(list(range(0, M // 2)) + list(range(K - (M - M // 2), K))))
        X = torch.zeros((M, K), dtype=torch.bfloat16)
        X[torch.arange(len(sel)), torch.tensor(sel)] = 1.0
        sels.append(sel)
        items.append((ql.quantize_pack(W.to(dev), g), X.to(dev), torch.empty((M, N), device=dev)))
    ql.GroupedGemm(items).run()
    torch.cuda.synchronize()
    for (_, _, y), w16f, sel in zip(items, w16s, sels):
        yy = y.cpu().numpy()
        for j, k in enumerate(sel):
            assert np.array_equal(yy[j], w16f[:, k]), k


def test_grouped_gemm_small_workspace_computes_nothing_for_split_entries(dev):
    """A workspace smaller than prepare asked for: split entries leave y untouched, the others are
    computed, and the call succeeds (no write outside the workspace)."""
    M = 512
    items = []
    for N, K in ((512, 4096), (256, 12288)):
        pw = ql.quantize_pack(synth.weight(N, K, seed=7 * N + K, device=dev), T)
        items.append((pw, synth.activations(M, K, seed=N, device=dev), torch.full((M, N), float("nan"), device=dev)))
    grp = ql.GroupedGemm(items)
    split = [p["splits"] > 1 for p in grp.plan]
    assert any(split) and grp.ws_bytes > 0
    st = ql.lib().qlinear_gemm_grouped(grp.descs.data_ptr(), grp.count, grp.total, M, grp.ws.data_ptr(), 16,
                                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    by_n = {p["N"]: p["splits"] > 1 for p in grp.plan}
    for pw, _, y in items:
        if by_n[pw.N]:
            assert torch.isnan(y).all()
        else:
            assert not torch.isnan(y).any()
