"""GPU parity: every kernel behind the C ABI against the CPU oracle (needs gfx950).

Bit-exact for codes, scales, packed bytes, unpacked codes and dequantized
weights; the products within max_n |dy| / ||y_row||_2 <= 2e-3 (GEMV, fp32
accumulation) and 1e-2 (GEMM, bf16 MFMA), plus tighter tripwires that the
measured error sits far below.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2
GEMV_TOL, GEMM_TOL = 2e-3, 1e-2
TRIP_GEMV, TRIP_GEMM = 1e-5, 1e-4  # normwise tripwires for the paths' actual arithmetic


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def grid_arg(N, grid, seed=0):
    """An int grid, or a seeded per-block table covering all three grids."""
    if grid != "mixed":
        return grid
    rng = np.random.default_rng(seed)
    nb = (N + 127) // 128
    t = rng.integers(0, 3, nb).astype(np.int8)
    t[: min(3, nb)] = [2, 0, 1][: min(3, nb)]
    return t


def oracle_grid(grid):
    return grid


SHAPES = [(1, 128), (3, 256), (64, 640), (129, 1280), (200, 2048), (1000, 4096), (130, 5120), (70, 384)]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
def test_quantize_pack_dequant_bit_exact(ora, dev, N, K, grid):
    note(f"quantize/pack N={N} K={K} grid={grid}")
    g = grid_arg(N, grid, seed=N + K)
    W = synth.weight(N, K, seed=100 + N + K)
    c_ref, s_ref = ora.quantize(W.numpy(), g)
    codes, scales = ql.quantize(W.to(dev), g)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(bits(scales), s_ref)
    pw = ql.pack(codes, scales, g)
    assert np.array_equal(pw.packed.cpu().numpy(), ora.pack(c_ref, g))
    assert np.array_equal(bits(pw.pscales), ora.pack_scales(s_ref, K))
    assert np.array_equal(ql.unpack(pw).cpu().numpy(), c_ref)
    assert np.array_equal(bits(ql.unpack_scales(pw)), s_ref)
    w32, w16 = ora.dequant(c_ref, s_ref)
    assert np.array_equal(ql.dequant(pw).cpu().numpy().view(np.uint32), w32.view(np.uint32))
    assert np.array_equal(bits(ql.dequant(pw, out_bf16=True)), w16)


def test_quantize_ties_and_zero_groups(ora, dev):
    s = 0.015625
    W = np.zeros((3, 256), np.float32)
    W[0, :9] = (np.arange(-9, 9, 2) / 2.0 * s).astype(np.float32)  # exact half-integer quotients
    W[0, 100] = 4 * s
    W[1, 128:] = 0.0  # an all-zero group
    W[1, :5] = [1e-40, -2e-41, 3e-39, 0, 5e-38]
    W[2] = synth.weight(1, 256, seed=5).numpy()[0]
    for g in (T, I2, I3):
        c_ref, s_ref = ora.quantize(W, g)
        codes, scales = ql.quantize(torch.from_numpy(W).to(dev), g)
        assert np.array_equal(codes.cpu().numpy(), c_ref)
        assert np.array_equal(bits(scales), s_ref)


def _gemv_case(ora, dev, N, K, grid, M, seed):
    g = grid_arg(N, grid, seed=seed)
    W = synth.weight(N, K, seed=seed)
    c_ref, s_ref = ora.quantize(W.numpy(), g)
    pw = ql.quantize_pack(W.to(dev), g)
    x = synth.activations(M, K, seed=seed + 1)
    y64 = ora.gemv(c_ref, s_ref, synth.bf16_bits(x))
    return pw, x.to(dev), y64, c_ref, s_ref


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
@pytest.mark.parametrize("M", [1, 3, 8, 16])
def test_gemv_parity(ora, dev, N, K, grid, M):
    note(f"gemv N={N} K={K} grid={grid} M={M}")
    pw, x, y64, _, _ = _gemv_case(ora, dev, N, K, grid, M, seed=N * 31 + K + M)
    y = ql.gemv(x, pw)
    torch.cuda.synchronize()
    err, normwise = ora.rel_err(y.cpu().numpy(), y64)
    assert err <= GEMV_TOL, (err, normwise)
    assert normwise <= TRIP_GEMV, normwise
    y2 = ql.gemv(x, pw)
    assert torch.equal(y, y2)  # bitwise deterministic


@pytest.mark.parametrize("grid", [T, I2, I3])
def test_gemv_one_hot_decodes_every_position(ora, dev, grid):
    """x = e_k gives y[n] = c[n,k] * s[n,k/128] exactly: the kernel's decode is bit-exact at every
    position residue (mod 80 for ternary chunks, mod 16 / 32 for 2-/3-bit words)."""
    N, K = 130, 1280
    note(f"one-hot grid={grid}")
    W = synth.weight(N, K, seed=77 + grid)
    c_ref, s_ref = ora.quantize(W.numpy(), grid)
    w32, _ = ora.dequant(c_ref, s_ref)
    pw = ql.quantize_pack(W.to(dev), grid)
    ks = list(range(0, 160)) + list(range(600, 700)) + list(range(K - 100, K))
    X = torch.zeros((len(ks), K), dtype=torch.bfloat16)
    for i, k in enumerate(ks):
        X[i, k] = 1.0
    X = X.to(dev)
    for i0 in range(0, len(ks), 8):
        y = ql.gemv(X[i0:i0 + 8].contiguous(), pw).cpu().numpy()
        for j, k in enumerate(ks[i0:i0 + 8]):
            assert np.array_equal(y[j], w32[:, k]), k


LARGE_M = 16  # qlinear_gemm runs the large-tile kernel (bf16 RNE(c*s) operands) from here on


def check_gemm(ora, y, y64, c_ref, s_ref, x, M):
    """The MFMA path's bar against the fp64 product; the tripwire against the product its operands
    define: below LARGE_M every product is exact (normwise 1e-4 of the fp64 product), from LARGE_M
    on the weights are bf16 RNE(c*s), and the result must match the oracle's bf16-weight product to
    fp32 summation error (normwise 1e-5)."""
    err, normwise = ora.rel_err(y, y64)
    assert err <= GEMM_TOL, (err, normwise)
    if M < LARGE_M:
        assert normwise <= TRIP_GEMM, normwise
    else:
        y16 = ora.gemv_w16(c_ref, s_ref, synth.bf16_bits(x.cpu()))
        _, nw16 = ora.rel_err(y, y16)
        assert nw16 <= TRIP_GEMV, nw16


@pytest.mark.parametrize("N,K", [(64, 128), (129, 1280), (1000, 4096), (70, 384), (256, 5120)])
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
@pytest.mark.parametrize("M", [1, 4, 8, 16, 17, 64, 100])
def test_gemm_parity(ora, dev, N, K, grid, M):
    note(f"gemm N={N} K={K} grid={grid} M={M}")
    pw, x, y64, c_ref, s_ref = _gemv_case(ora, dev, N, K, grid, M, seed=N * 7 + K + M)
    y = ql.gemm(x, pw)
    torch.cuda.synchronize()
    check_gemm(ora, y.cpu().numpy(), y64, c_ref, s_ref, x, M)


BIG_GEMM_CASES = [(64, 128, 128), (129, 1280, 200), (1000, 4096, 128), (70, 384, 384), (256, 5120, 256),
                  (520, 1920, 130), (300, 12288, 128), (300, 4096, 512), (64, 128, 256), (520, 1920, 300),
                  (129, 1280, 257), (1000, 4096, 256)]


@pytest.mark.parametrize("N,K,M", BIG_GEMM_CASES)
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
def test_gemm_large_batch_parity(ora, dev, N, K, M, grid):
    """Batches of 128 tokens and more (the large-tile kernel): ragged token tiles (M = 130, 200,
    257, 300), rows past N, mixed grid blocks, long rows and K splits."""
    note(f"gemm large batch N={N} K={K} grid={grid} M={M}")
    pw, x, y64, c_ref, s_ref = _gemv_case(ora, dev, N, K, grid, M, seed=N * 5 + K + M)
    y = ql.gemm(x, pw)
    torch.cuda.synchronize()
    check_gemm(ora, y.cpu().numpy(), y64, c_ref, s_ref, x, M)


@pytest.mark.parametrize("N,K", [(300, 1280), (256, 4096), (130, 384)])
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
@pytest.mark.parametrize("M", [16, 100, 256])
def test_gemm_large_tile_one_hot(ora, dev, N, K, grid, M):
    """x rows = e_k: the large-tile kernel returns bf16 RNE(c*s) of every weight exactly (one
    exact product per output), at every position residue of the decoders and across tiles."""
    note(f"gemm one-hot N={N} K={K} grid={grid} M={M}")
    g = grid_arg(N, grid, seed=N + K)
    W = synth.weight(N, K, seed=31 * N + K)
    c_ref, s_ref = ora.quantize(W.numpy(), g)
    _, w16 = ora.dequant(c_ref, s_ref)
    w16f = (w16.astype(np.uint32) << 16).view(np.float32)
    pw = ql.quantize_pack(W.to(dev), g)
    ks = sorted(set(list(range(0, min(K, 160))) + list(range(max(0, K - 100), K))))
    for i0 in range(0, len(ks), M):
        sel = ks[i0:i0 + M]
        X = torch.zeros((M, K), dtype=torch.bfloat16)
        X[torch.arange(len(sel)), torch.tensor(sel)] = 1.0
        y = ql.gemm(X.to(dev), pw).cpu().numpy()
        for j, k in enumerate(sel):
            assert np.array_equal(y[j], w16f[:, k]), (k, np.flatnonzero(y[j] != w16f[:, k])[:5])
        assert not y[len(sel):].any()


def test_grouped_gemv_parity(ora, dev):
    note("grouped gemv")
    cases = [(256, 4096, "mixed"), (1024, 4096, I3), (128, 12288, T), (3, 640, I2), (1000, 2048, T)]
    for M in (1,):
        items, refs = [], []
        for i, (N, K, grid) in enumerate(cases):
            pw, x, y64, _, _ = _gemv_case(ora, dev, N, K, grid, M, seed=500 + i + M)
            y = torch.full((M, N), float("nan"), device=dev)
            items.append((pw, x, y))
            refs.append(y64)
        grp = ql.GroupedGemv(items)
        grp.run()
        torch.cuda.synchronize()
        for (pw, x, y), y64 in zip(items, refs):
            err, normwise = ora.rel_err(y.cpu().numpy(), y64)
            assert err <= GEMV_TOL and normwise <= TRIP_GEMV, (pw.N, pw.K, err, normwise)


def test_grouped_gemv_repeats_and_matches_single_launches(ora, dev):
    """Tasks are drawn from an atomic counter in longest-first order; every launch leaves the
    counter zero, repeated launches are bitwise identical, and each product equals the
    single-matrix launch bitwise (the per-row arithmetic does not depend on which wave runs it)."""
    note("grouped gemv repeated")
    cases = [(64, 4096, T), (300, 12288, "mixed"), (1, 640, I3), (4096, 4096, I2), (200, 1280, T), (128, 12288, I3)]
    items = []
    for i, (N, K, grid) in enumerate(cases):
        pw, x, _, _, _ = _gemv_case_dev(dev, N, K, grid, seed=900 + i)
        items.append((pw, x, torch.full((1, N), float("nan"), device=dev)))
    grp = ql.GroupedGemv(items)
    outs = []
    for _ in range(3):
        grp.run()
        torch.cuda.synchronize()
        assert int(grp.sched.abs().sum().item()) == 0
        outs.append([y.clone() for _, _, y in items])
    for (pw, x, y), y1, y2 in zip(items, outs[1], outs[2]):
        assert torch.equal(y, y1) and torch.equal(y, y2)
        assert torch.equal(y, ql.gemv(x, pw))


def _gemv_case_dev(dev, N, K, grid, seed):
    g = grid_arg(N, grid, seed=seed)
    W = synth.weight(N, K, seed=seed, device=dev)
    return ql.quantize_pack(W, g), synth.activations(1, K, seed=seed + 1, device=dev), None, None, None


def test_workload_linear2048_i2(ora, dev):
    """One 2048x2048 linear, uniform 2-bit grid, batch 1, at full size."""
    note("workload linear2048_i2")
    pw, x, y64, _, _ = _gemv_case(ora, dev, 2048, 2048, I2, 1, seed=synth.weight_seed(0, 0, 0))
    err, normwise = ora.rel_err(ql.gemv(x, pw).cpu().numpy(), y64)
    assert err <= GEMV_TOL and normwise <= TRIP_GEMV


def test_grouped_gemv_batch_above_one_goes_to_batched_kernel(ora, dev):
    """M = 4 in a grouped launch (one token group of four) meets the GEMV bar."""
    pw, x, y64, _, _ = _gemv_case(ora, dev, 128, 640, T, 4, seed=9)
    y = torch.full((4, 128), float("nan"), device=dev)
    ql.GroupedGemv([(pw, x, y)]).run()
    torch.cuda.synchronize()
    err, normwise = ora.rel_err(y.cpu().numpy(), y64)
    assert err <= GEMV_TOL and normwise <= TRIP_GEMV, (err, normwise)
