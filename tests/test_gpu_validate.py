"""The data checks (qlinear_validate_codes / qlinear_validate_packed), needs gfx950.

Valid weights count nothing; planted faults are counted exactly: codes outside
their row's grid, a ternary byte above 242 (a base-3 byte of five trits is at
most 242; ThinkBit summary page, onedev.kr/papers/1416, section "How it works"
for the grids), padding that does not code c = 0 (rows past N, trits past K),
and a block grid id that is not a grid.
"""
import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def table(N):
    t = np.array([T, I3, I2] * ((N + 383) // 384), np.int8)[: (N + 127) // 128]
    return t


@pytest.mark.parametrize("N,K", [(130, 384), (70, 1280), (256, 4096), (1, 128)])
@pytest.mark.parametrize("grid", [T, I2, I3, "mixed"])
def test_valid_weights_count_nothing(dev, N, K, grid):
    g = table(N) if grid == "mixed" else grid
    W = synth.weight(N, K, seed=N + K, device=dev)
    codes, scales = ql.quantize(W, g)
    assert not ql.validate_codes(codes, g).any()
    pw = ql.pack(codes, scales, g)
    assert not ql.validate_packed(pw).any()


def test_codes_outside_the_grid(dev):
    N, K = 130, 256
    g = table(N)  # blocks: ternary, 3-bit
    codes = torch.zeros((N, K), dtype=torch.int8, device=dev)
    codes[0, 5] = 2    # ternary row: outside {-1, 0, 1}
    codes[1, 7] = -2   # ternary row: outside
    codes[129, 0] = 3  # 3-bit row: inside {-4..3}
    codes[129, 1] = -5  # 3-bit row: outside
    codes[128, 9] = 4   # outside
    got = ql.validate_codes(codes, g)
    assert list(got) == [4, 0, 0, 0]
    assert list(ql.validate_codes(codes, I3)) == [2, 0, 0, 0]  # only -5 and 4 fall outside 3-bit
    bad = g.copy()
    bad[1] = 7
    assert list(ql.validate_codes(codes, bad)) == [2, 0, 1, 0]  # block 1 skipped and counted


def test_packed_faults(dev):
    N, K = 130, 384  # rows 130..191 pad the last slab; ternary rows hold 400 trits (384..399 pad)
    W = synth.weight(N, K, seed=9, device=dev)
    pw = ql.quantize_pack(W, T)
    assert not ql.validate_packed(pw).any()
    rb = ql.row_bytes(T, K)  # 80
    p0 = pw.packed.clone()

    def at(n, j):  # byte j of row n in the slab interleave
        return (n // 64) * 64 * rb + (j // 16) * 1024 + (n % 64) * 16 + (j % 16)

    pw.packed[at(3, 10)] = 250                 # a ternary byte above 242
    assert list(ql.validate_packed(pw)) == [1, 0, 0, 0]
    pw.packed.copy_(p0)
    pw.packed[at(5, 77)] = 0                   # inputs 385..389: padding, all five digits c = -1
    assert list(ql.validate_packed(pw)) == [0, 5, 0, 0]
    pw.packed.copy_(p0)
    pw.packed[at(140, 3)] = 121 + 1            # a padding row: one digit off c = 0
    assert list(ql.validate_packed(pw)) == [0, 1, 0, 0]
    pw.packed.copy_(p0)
    assert not ql.validate_packed(pw).any()


def test_packed_padding_rows_and_block_grids(dev):
    N, K = 130, 256
    g = np.array([I2, I3], np.int8)
    W = synth.weight(N, K, seed=10, device=dev)
    pw = ql.quantize_pack(W, g)
    assert not ql.validate_packed(pw).any()
    off = pw.blk_off.cpu().numpy()
    p0 = pw.packed.clone()
    # block 1 (3-bit) holds one slab, rows 128..191, of which 130..191 pad past N = 130
    pw.packed[int(off[1]) + 12 * 16] ^= 0x01  # row 140, input 0: code u 4 -> 5, off c = 0
    assert list(ql.validate_packed(pw)) == [0, 1, 0, 0]
    pw.packed.copy_(p0)
    pw.blk_grid[1] = 9
    assert list(ql.validate_packed(pw)) == [0, 0, 1, 0]
