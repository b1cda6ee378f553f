"""GPU parity of the whole Qwen3-8B decode pass, in the launches the benchmark times (needs gfx950).

All 36 layers x 7 linears (252 matrices, mixed grids) are generated with the same
seeds, quantized and packed on the GPU, and run as ONE grouped batch-1 launch.
The oracle recomputes 24 seeded rows of every linear of four layers (first,
last and two between).  Every one of the 252 outputs is also compared bitwise
with a launch of that matrix alone: without split-K each 64-row slab is summed
by one wave in a fixed order, whatever else shares the launch, so grouping must
not change a bit.  The dependency-respecting variant (four grouped launches per
layer, split-K on) is checked on two layers at M = 1 and 4 against the oracle.
Tolerance: max_n |dy| / ||y_row|| <= 2e-3, with each sampled row set's norm
scaled to the full row count, and the normwise tripwire 1e-5.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import configs
from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

TOL, TRIP = 2e-3, 1e-5
WL = "qwen3_8b_pass"
SAMPLED_LAYERS = (0, 11, 24, 35)
ROWS = 24


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def oracle_rows(ora, W_gpu, rows, grid, x_bits):
    """Oracle y for the given rows of W, each row quantized by the oracle on its block's grid."""
    Wr = W_gpu[torch.from_numpy(rows).to(W_gpu.device)].cpu().numpy()
    gtab = np.full((W_gpu.shape[0] + 127) // 128, grid, np.int8) if np.isscalar(grid) else np.asarray(grid, np.int8)
    row_grid = gtab[rows // 128]
    codes = np.empty(Wr.shape, np.int8)
    scales = np.empty((len(rows), Wr.shape[1] // 128), np.uint16)
    for g in np.unique(row_grid):
        sel = row_grid == g
        codes[sel], scales[sel] = ora.quantize(Wr[sel], int(g))
    return ora.gemv(codes, scales, x_bits)


def check_rows(yg, y64, N):
    d = np.abs(yg - y64).max(axis=1)
    full_norm = np.linalg.norm(y64, axis=1) * np.sqrt(N / y64.shape[1])
    err = float((d / full_norm).max())
    nw = float(np.linalg.norm(yg - y64) / np.linalg.norm(y64))
    assert err <= TOL and nw <= TRIP, (err, nw)


@pytest.fixture(scope="module")
def full_pass(dev):
    """Packed matrices of the 8B pass with the seeds, grids and activations of the benchmark."""
    wl = configs.WORKLOADS[WL]
    wi = list(configs.WORKLOADS).index(WL)
    note(f"packing {wl.layers} layers of {WL}")
    items, meta, xs = [], [], {}
    for layer in range(wl.layers):
        alloc = synth.allocation(wl, layer)
        for slot in ("attn", "o", "mlp", "down"):
            K = next(l.K for l in wl.linears if l.x_slot == slot)
            xs[(layer, slot)] = synth.activations(1, K, synth.x_seed(wi, layer, slot, 1), device=dev)
        for mi, lin in enumerate(wl.linears):
            W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, layer, mi), device=dev)
            pw = ql.quantize_pack(W, alloc[lin.name])
            del W
            items.append((pw, xs[(layer, lin.x_slot)], torch.full((1, lin.N), float("nan"), device=dev)))
            meta.append((layer, mi, lin, alloc[lin.name]))
    torch.cuda.synchronize()
    return wl, wi, items, meta


def test_full_pass_single_grouped_launch(ora, dev, full_pass):
    wl, wi, items, meta = full_pass
    note(f"one grouped launch over {len(items)} matrices")
    ql.GroupedGemv(items).run()
    torch.cuda.synchronize()
    for (pw, x, y), (layer, mi, lin, grid) in zip(items, meta):
        assert bool(torch.isfinite(y).all()), (layer, lin.name)
    rng = np.random.default_rng(8036)
    for (pw, x, y), (layer, mi, lin, grid) in zip(items, meta):
        if layer not in SAMPLED_LAYERS:
            continue
        note(f"8B pass layer {layer}: {lin.name} {lin.N}x{lin.K} against the oracle")
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, layer, mi), device=dev)
        rows = np.sort(rng.choice(lin.N, size=ROWS, replace=False))
        y64 = oracle_rows(ora, W, rows, grid, synth.bf16_bits(x.cpu()))
        check_rows(y[:, torch.from_numpy(rows).to(dev)].cpu().numpy(), y64, lin.N)
        del W
    note("every matrix alone, bitwise against its slice of the grouped launch")
    for (pw, x, y), (layer, mi, lin, grid) in zip(items, meta):
        y1 = torch.full_like(y, float("nan"))
        ql.GroupedGemv([(pw, x, y1)]).run()
        torch.cuda.synchronize()
        assert torch.equal(y, y1), (layer, lin.name)


@pytest.mark.parametrize("M", [1, 4])
def test_full_pass_layered_split_launches(ora, dev, full_pass, M):
    """Four grouped launches per layer in model order with split-K on, as the layered pass runs."""
    wl, wi, items1, meta = full_pass
    rng = np.random.default_rng(8100 + M)
    for layer in (0, 35):
        xs = {}
        for slot in ("attn", "o", "mlp", "down"):
            K = next(l.K for l in wl.linears if l.x_slot == slot)
            xs[slot] = synth.activations(M, K, synth.x_seed(wi, layer, slot, M), device=dev)
        for slot in ("attn", "o", "mlp", "down"):
            sel = [i for i, m in enumerate(meta) if m[0] == layer and m[2].x_slot == slot]
            its = [(items1[i][0], xs[slot], torch.full((M, meta[i][2].N), float("nan"), device=dev)) for i in sel]
            grp = ql.GroupedGemv(its, split="auto")
            note(f"layered layer {layer} {slot} M={M}: kparts {grp.kparts}")
            grp.run()
            torch.cuda.synchronize()
            for (pw, x, y), i in zip(its, sel):
                _, mi, lin, grid = meta[i]
                W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, layer, mi), device=dev)
                rows = np.sort(rng.choice(lin.N, size=ROWS, replace=False))
                y64 = oracle_rows(ora, W, rows, grid, synth.bf16_bits(x.cpu()))
                check_rows(y[:, torch.from_numpy(rows).to(dev)].cpu().numpy(), y64, lin.N)
                del W
