"""GPU parity of the 4-bit container baseline (needs gfx950).

Container bytes, unpacked codes and the container -> native converter are
checked bit-exactly against the oracle; the container GEMV against the oracle's
product within the GEMV contract (max_n |dy| / ||y||_2 <= 2e-3, normwise
tripwire 1e-5), with one-hot activations checking the decode exactly.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import configs
from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2
GEMV_TOL, TRIP_GEMV = 2e-3, 1e-5
SHAPES = [(1, 128), (3, 256), (64, 640), (129, 1280), (200, 2048), (1000, 4096), (130, 5120), (70, 384)]


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def grid_arg(N, grid, seed=0):
    if grid != "mixed":
        return grid
    rng = np.random.default_rng(seed)
    t = rng.integers(0, 3, (N + 127) // 128).astype(np.int8)
    t[: min(3, len(t))] = [2, 0, 1][: min(3, len(t))]
    return t


def quantized(ora, N, K, grid, seed):
    W = synth.weight(N, K, seed=seed)
    return ora.quantize(W.numpy(), grid)


def to_dev(dev, codes, scales):
    return (torch.from_numpy(codes).to(dev),
            torch.from_numpy(scales.view(np.int16)).view(torch.bfloat16).to(dev))


@pytest.mark.parametrize("N,K", SHAPES)
def test_c4_pack_unpack_bit_exact(ora, dev, N, K):
    note(f"c4 pack N={N} K={K}")
    rng = np.random.default_rng(N * 7 + K)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    scales = np.zeros((N, K // 128), np.uint16)
    cw = ql.c4_pack(*to_dev(dev, codes, scales))
    assert cw.c4.numel() == ora.lib().ora_c4_bytes(N, K)
    assert np.array_equal(cw.c4.cpu().numpy(), ora.c4_pack(codes))
    assert np.array_equal(ql.c4_unpack(cw).cpu().numpy(), codes)


@pytest.mark.parametrize("N,K", [(3, 256), (129, 1280), (200, 2048), (130, 5120), (70, 384)])
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
def test_c4_to_packed_equals_native_pack(ora, dev, N, K, grid):
    note(f"c4 -> packed N={N} K={K} grid={grid}")
    g = grid_arg(N, grid, seed=N + K)
    codes, scales = quantized(ora, N, K, g, 300 + N + K)
    cw = ql.c4_pack(*to_dev(dev, codes, scales))
    pw = ql.c4_to_packed(cw, g)
    assert np.array_equal(pw.packed.cpu().numpy(), ora.pack(codes, g))
    assert np.array_equal(ql.unpack(pw).cpu().numpy(), codes)


@pytest.mark.parametrize("N,K", SHAPES)
@pytest.mark.parametrize("grid", [T, I3, "mixed"])
def test_c4_gemv_matches_oracle(ora, dev, N, K, grid):
    note(f"c4 gemv N={N} K={K} grid={grid}")
    g = grid_arg(N, grid, seed=N * 3 + K)
    codes, scales = quantized(ora, N, K, g, 500 + N + K)
    cw = ql.c4_pack(*to_dev(dev, codes, scales))
    x = synth.activations(1, K, seed=N + 2 * K)
    y = ql.c4_gemv(x.to(dev), cw)
    y64 = ora.gemv(codes, scales, synth.bf16_bits(x))
    err, nw = ora.rel_err(y.cpu().numpy(), y64)
    assert err <= GEMV_TOL and nw <= TRIP_GEMV, (err, nw)


def test_c4_gemv_full_code_range(ora, dev):
    """Codes over the whole container range -8..7 (wider than any ThinkBit grid)."""
    N, K = 200, 1280
    rng = np.random.default_rng(11)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    scales = ora.f32_to_bf16(rng.uniform(0.001, 0.05, (N, K // 128)).astype(np.float32))
    cw = ql.c4_pack(*to_dev(dev, codes, scales))
    x = synth.activations(1, K, seed=12)
    y = ql.c4_gemv(x.to(dev), cw)
    y64 = ora.gemv(codes, scales, synth.bf16_bits(x))
    err, nw = ora.rel_err(y.cpu().numpy(), y64)
    assert err <= GEMV_TOL and nw <= TRIP_GEMV, (err, nw)


def test_c4_gemv_one_hot_decode_exact(ora, dev):
    """x = e_k gives y[n] = c[n,k] * s[n,k/128] exactly: every position in a 32-input
    chunk, the first and last group, and the last input."""
    N, K = 130, 640
    rng = np.random.default_rng(13)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    scales = ora.f32_to_bf16(rng.uniform(0.001, 0.05, (N, K // 128)).astype(np.float32))
    cw = ql.c4_pack(*to_dev(dev, codes, scales))
    w32, _ = ora.dequant(codes, scales)
    ks = list(range(32)) + [100, 127, 128, 300, 511, 512, 600, 639]
    one = np.uint16(0x3F80)  # bf16 1.0
    for k in ks:
        xb = np.zeros(K, np.uint16)
        xb[k] = one
        x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).view(1, K).to(dev)
        y = ql.c4_gemv(x, cw).cpu().numpy()[0]
        assert np.array_equal(y.view(np.uint32), w32[:, k].view(np.uint32)), k


def test_c4_grouped_repeats_and_matches_single_launches(ora, dev):
    shapes = [(200, 2048), (64, 640), (1000, 4096), (70, 384), (130, 5120)]
    items, singles = [], []
    for i, (N, K) in enumerate(shapes):
        codes, scales = quantized(ora, N, K, grid_arg(N, "mixed", i), 700 + i)
        cw = ql.c4_pack(*to_dev(dev, codes, scales))
        x = synth.activations(1, K, seed=800 + i).to(dev)
        items.append((cw, x, torch.full((1, N), float("nan"), device=dev)))
        singles.append(ql.c4_gemv(x, cw))
    grp = ql.GroupedGemv(items)
    for rep in range(3):
        for _, _, y in items:
            y.fill_(float("nan"))
        grp.run()
        torch.cuda.synchronize()
        assert not grp.sched.any().item(), rep
        for (_, _, y), ys in zip(items, singles):
            assert torch.equal(y, ys), rep


def test_c4_qwen3_1p7b_layer_every_row(ora, dev):
    """A Qwen3-1.7B layer (mixed grids) as containers in one grouped launch; every row."""
    wl = configs.WORKLOADS["qwen3_1p7b_layer"]
    wi = list(configs.WORKLOADS).index(wl.name)
    alloc = synth.allocation(wl, 0)
    xs = {slot: synth.activations(1, next(l.K for l in wl.linears if l.x_slot == slot),
                                  synth.x_seed(wi, 0, slot, 1)) for slot in ("attn", "o", "mlp", "down")}
    items, refs = [], []
    for mi, lin in enumerate(wl.linears):
        note(f"1.7B layer (containers): {lin.name} {lin.N}x{lin.K}")
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, 0, mi))
        c, s = ora.quantize(W.numpy(), alloc[lin.name])
        refs.append(ora.gemv(c, s, synth.bf16_bits(xs[lin.x_slot])))
        codes, scales = ql.quantize(W.to(dev), alloc[lin.name])
        items.append((ql.c4_pack(codes, scales), xs[lin.x_slot].to(dev), torch.empty((1, lin.N), device=dev)))
    ql.GroupedGemv(items).run()
    torch.cuda.synchronize()
    for (_, _, y), y64, lin in zip(items, refs, wl.linears):
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= GEMV_TOL and nw <= TRIP_GEMV, (lin.name, err, nw)
