"""GPU parity at the workloads' full sizes (needs gfx950).

Each matrix is generated, quantized and packed on the GPU at its real shape,
in the launch the benchmark uses (grouped GEMV at batch 1, the MFMA path above
it).  The CPU oracle recomputes every row of the 1.7B layer, and a seeded
sample of rows of the larger matrices (the oracle cannot afford whole 8B/14B
layers per test).  Tolerances: max_n |dy| / ||y_row|| <= 2e-3 (GEMV) and 1e-2
(GEMM), both measured against the sampled rows' norm scaled to the full row
count; plus the normwise tripwires of the small-shape tests.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import configs
from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

GEMV_TOL, GEMM_TOL = 2e-3, 1e-2
TRIP_GEMV, TRIP_GEMM = 1e-5, 1e-4


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def wl_index(name):
    return list(configs.WORKLOADS).index(name)


def oracle_rows(ora, W_gpu, rows, grid, x_bits, w16=False):
    """Oracle y for the given rows of W (quantized on the CPU by the oracle, per row's grid);
    w16: the product with bf16 RNE(c*s) weights instead of the exact fp32 ones."""
    idx = torch.from_numpy(rows).to(W_gpu.device)
    Wr = W_gpu[idx].cpu().numpy()
    gtab = np.full((W_gpu.shape[0] + 127) // 128, grid, np.int8) if np.isscalar(grid) else np.asarray(grid, np.int8)
    row_grid = gtab[rows // 128]
    codes = np.empty(Wr.shape, np.int8)
    scales = np.empty((len(rows), Wr.shape[1] // 128), np.uint16)
    for g in np.unique(row_grid):
        sel = row_grid == g
        c, s = ora.quantize(Wr[sel], int(g))
        codes[sel], scales[sel] = c, s
    return ora.gemv_w16(codes, scales, x_bits) if w16 else ora.gemv(codes, scales, x_bits)


def check_rows(y_gpu_rows, y64, N, tol, trip):
    """Tolerance on sampled rows, with each token row's norm scaled to the full row count."""
    d = np.abs(y_gpu_rows - y64).max(axis=1)
    full_norm = np.linalg.norm(y64, axis=1) * np.sqrt(N / y64.shape[1])
    err = float((d / full_norm).max())
    nw = float(np.linalg.norm(y_gpu_rows - y64) / np.linalg.norm(y64))
    assert err <= tol and nw <= trip, (err, nw)
    return err, nw


def test_config1_qwen3_1p7b_layer_every_row(ora, dev):
    """One Qwen3-1.7B layer, mixed grids (q, k 3-bit), batch 1, one grouped launch; every row."""
    wl = configs.WORKLOADS["qwen3_1p7b_layer"]
    wi = wl_index(wl.name)
    alloc = synth.allocation(wl, 0)
    xs = {slot: synth.activations(1, next(l.K for l in wl.linears if l.x_slot == slot),
                                  synth.x_seed(wi, 0, slot, 1)) for slot in ("attn", "o", "mlp", "down")}
    items, refs = [], []
    for mi, lin in enumerate(wl.linears):
        note(f"1.7B layer: {lin.name} {lin.N}x{lin.K}")
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, 0, mi))
        c, s = ora.quantize(W.numpy(), alloc[lin.name])
        refs.append(ora.gemv(c, s, synth.bf16_bits(xs[lin.x_slot])))
        pw = ql.quantize_pack(W.to(dev), alloc[lin.name])
        items.append((pw, xs[lin.x_slot].to(dev), torch.full((1, lin.N), float("nan"), device=dev)))
    ql.GroupedGemv(items).run()
    torch.cuda.synchronize()
    for (pw, x, y), y64, lin in zip(items, refs, wl.linears):
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= GEMV_TOL and nw <= TRIP_GEMV, (lin.name, err, nw)


@pytest.mark.parametrize("layer", [0, 39])
@pytest.mark.parametrize("M,path", [(1, "grouped"), (4, "grouped"), (16, "grouped"), (4, "mfma"), (16, "mfma")])
def test_config3_qwen3_14b_layer_sampled(ora, dev, layer, M, path):
    """A Qwen3-14B layer at full size (down_proj K = 17408 included), mixed grids, 48 seeded rows
    per matrix.  path "grouped": the grouped launch the benchmark times (the decode GEMV with one
    and four token groups; GEMV bar).  path "mfma": qlinear_gemm, the small-batch LDS-tile kernel
    at M = 4 and the large-tile kernel at M = 16 (GEMM bar)."""
    wl = configs.WORKLOADS["qwen3_14b_stack"]
    wi = wl_index(wl.name)
    alloc = synth.allocation(wl, layer)
    rng = np.random.default_rng(1000 * layer + M)
    xs = {slot: synth.activations(M, next(l.K for l in wl.linears if l.x_slot == slot),
                                  synth.x_seed(wi, layer, slot, M), device=dev) for slot in ("attn", "o", "mlp", "down")}
    mats = []
    for mi, lin in enumerate(wl.linears):
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, layer, mi), device=dev)
        pw = ql.quantize_pack(W, alloc[lin.name])
        mats.append((lin, W, pw))
    note(f"14B layer {layer} M={M} path={path}")
    if path == "grouped":
        items = [(pw, xs[lin.x_slot], torch.full((M, lin.N), float("nan"), device=dev)) for lin, _, pw in mats]
        ql.GroupedGemv(items).run()
        ys = [y for _, _, y in items]
    else:
        ys = [ql.gemm(xs[lin.x_slot], pw) for lin, _, pw in mats]
    torch.cuda.synchronize()
    tol, trip = (GEMV_TOL, TRIP_GEMV) if path == "grouped" else (GEMM_TOL, TRIP_GEMM)
    for (lin, W, pw), y in zip(mats, ys):
        note(f"14B layer {layer} M={M} {path}: {lin.name} {lin.N}x{lin.K}")
        rows = np.sort(rng.choice(lin.N, size=48, replace=False))
        y64 = oracle_rows(ora, W, rows, alloc[lin.name], synth.bf16_bits(xs[lin.x_slot].cpu()))
        yg = y[:, torch.from_numpy(rows).to(dev)].cpu().numpy()
        if path == "mfma" and M >= 16:
            # large-tile kernel: bf16 RNE(c*s) operands; the bar against the exact product,
            # the tripwire against the bf16-weight product
            check_rows(yg, y64, lin.N, tol, 1.0)
            y16 = oracle_rows(ora, W, rows, alloc[lin.name], synth.bf16_bits(xs[lin.x_slot].cpu()), w16=True)
            check_rows(yg, y16, lin.N, tol, TRIP_GEMV)
        else:
            check_rows(yg, y64, lin.N, tol, trip)


@pytest.mark.parametrize("grid", ["T", "I2", "I3", "mixed"])
@pytest.mark.parametrize("M", [64, 256, 512])
def test_config4_qwen3_8b_layer_gemm_sampled(ora, dev, grid, M):
    """A Qwen3-8B layer's linears through qlinear_gemm at M in {64, 256, 512}, each grid and
    mixed; 32 seeded rows per matrix.  The bar (1e-2) against the exact product; the tripwire
    against the bf16-weight product that the large-tile kernel's operands define."""
    wl = configs.WORKLOADS["qwen3_8b_gemm"]
    wi = wl_index(wl.name)
    alloc = synth.allocation(wl, 0)
    g_of = {"T": 0, "I2": 1, "I3": 2}
    rng = np.random.default_rng(7 * M + len(grid))
    xs = {K: synth.activations(M, K, synth.seed_of(3, wi, K, M), device=dev) for K in (4096, 12288)}
    for mi, lin in enumerate(wl.linears):
        note(f"8B layer gemm {grid} M={M}: {lin.name}")
        g = alloc[lin.name] if grid == "mixed" else g_of[grid]
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, 0, mi), device=dev)
        pw = ql.quantize_pack(W, g)
        y = ql.gemm(xs[lin.K], pw)
        torch.cuda.synchronize()
        rows = np.sort(rng.choice(lin.N, size=32, replace=False))
        y64 = oracle_rows(ora, W, rows, g, synth.bf16_bits(xs[lin.K].cpu()))
        yg = y[:, torch.from_numpy(rows).to(dev)].cpu().numpy()
        check_rows(yg, y64, lin.N, GEMM_TOL, 1.0)
        y16 = oracle_rows(ora, W, rows, g, synth.bf16_bits(xs[lin.K].cpu()), w16=True)
        check_rows(yg, y16, lin.N, GEMM_TOL, TRIP_GEMV)
        del W, pw, y
