"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks one oracle function against a fact fixed by the pages or by
mathematics: brute force over the grid with exact rationals, closed forms,
exact sums, invariants, or a library routine (torch's bf16 rounding, Python's
base-3 integer parsing, a float64 matmul).  A plausible slip in the oracle (a
dropped term, a wrong sign, a swapped index, a wrong bit position) fails at
least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import synth

T, I2, I3 = 0, 1, 2
GRIDS = {T: (-1, 1), I2: (-2, 1), I3: (-4, 3)}  # summary page, "How it works"


def torch_bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(
        np.uint16)


def bf16_value(bits):
    return np.asarray(bits, dtype=np.uint32).astype(np.uint32) << 16


def f32_of_bf16(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_rne_matches_torch(ora):
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # denormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32),
        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    finite = np.isfinite(vals) | np.isinf(vals)
    mine = ora.f32_to_bf16(vals)
    ref = torch_bf16_bits(vals)
    assert np.array_equal(mine[finite & ~np.isnan(vals)], ref[finite & ~np.isnan(vals)])
    nan = np.isnan(vals)
    assert np.all(mine[nan] == 0x7FC0)


def test_bf16_golden_cases(ora):
    # tests/golden/bf16_rne.txt: IEEE-754 round-to-nearest-even cases worked by hand
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    f = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(np.float32)
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint16)
    assert np.array_equal(ora.f32_to_bf16(f), want)
    assert np.array_equal(ora.bf16_to_f32(want).view(np.uint32), want.astype(np.uint32) << 16)


# ---------------------------------------------------------------- quantizer
def brute_force_quantize(W, grid):
    """Scale from torch's bf16 rounding of max|w|/|c_min|; code = nearest grid point by exact
    rational distance, ties to the even code (the argmin formulation, not round-then-clamp)."""
    cmin, cmax = GRIDS[grid]
    N, K = W.shape
    G = K // 128
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, G), np.uint16)
    for n in range(N):
        for g in range(G):
            w = W[n, g * 128:(g + 1) * 128]
            a = np.float32(np.max(np.abs(w)))
            sb = torch_bf16_bits(np.array([a / np.float32(-cmin)], np.float32))[0]
            scales[n, g] = sb
            s = Fraction(float(f32_of_bf16(np.array([sb]))[0]))
            for i in range(128):
                if s == 0:
                    codes[n, g * 128 + i] = 0
                    continue
                wf = Fraction(float(w[i]))
                best = None
                for c in range(cmin, cmax + 1):
                    d = abs(wf - c * s)
                    if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                        best = (d, c)
                codes[n, g * 128 + i] = best[1]
    return codes, scales


@pytest.mark.parametrize("grid", [T, I2, I3])
def test_quantize_brute_force_random(ora, grid):
    W = synth.weight(3, 256, seed=11 + grid).numpy()
    c, s = ora.quantize(W, grid)
    cb, sb = brute_force_quantize(W, grid)
    assert np.array_equal(s, sb)
    assert np.array_equal(c, cb)


@pytest.mark.parametrize("grid", [T, I2, I3])
def test_quantize_brute_force_adversarial(ora, grid):
    cmin, cmax = GRIDS[grid]
    rng = np.random.default_rng(5 + grid)
    rows = []
    # exact half-integer multiples of the group scale (ties), the max on either sign, zeros
    for sign in (1.0, -1.0):
        s = 0.015625  # exact in bf16
        amax = s * (-cmin)
        w = np.zeros(128, np.float32)
        w[0] = sign * amax
        halves = np.arange(cmin * 2 - 1, cmax * 2 + 2) / 2.0
        w[1:1 + len(halves)] = (halves * s).astype(np.float32)
        w[40:80] = rng.uniform(-amax, amax, 40).astype(np.float32)
        rows.append(w)
    rows.append(np.zeros(128, np.float32))  # all-zero group -> s = 0, c = 0
    w = np.zeros(128, np.float32)
    w[7] = 1e-40  # a denormal maximum
    w[9] = -3e-41
    rows.append(w)
    W = np.stack(rows)
    c, s = ora.quantize(W, grid)
    cb, sb = brute_force_quantize(W, grid)
    assert np.array_equal(s, sb)
    assert np.array_equal(c, cb)
    assert s[2, 0] == 0 and np.all(c[2] == 0)


@pytest.mark.parametrize("grid", [T, I2, I3])
def test_quantize_error_bound_and_range(ora, grid):
    cmin, cmax = GRIDS[grid]
    W = synth.weight(16, 512, seed=3).numpy()
    c, s = ora.quantize(W, grid)
    assert c.min() >= cmin and c.max() <= cmax
    sf = np.repeat(f32_of_bf16(s).astype(np.float64), 128, axis=1)
    q = W.astype(np.float64) / sf
    inside = (q >= cmin - 0.5) & (q <= cmax + 0.5)
    err = np.abs(W.astype(np.float64) - c * sf)
    assert np.all(err[inside] <= sf[inside] / 2)


@pytest.mark.parametrize("grid", [T, I2, I3])
def test_requantize_reproduces_codes(ora, grid):
    """Re-rounding with the stored scales reproduces the stored codes (the invariant the k-quant
    calibration page reports for all 248 tensors, section "Open question")."""
    W = synth.weight(8, 384, seed=21).numpy()
    c, s = ora.quantize(W, grid)
    assert np.array_equal(ora.requantize(W, s, grid), c)
    w32, _ = ora.dequant(c, s)
    assert np.array_equal(ora.requantize(w32, s, grid), c)
    # arbitrary codes and arbitrary positive bf16 scales
    rng = np.random.default_rng(9)
    cmin, cmax = GRIDS[grid]
    cr = rng.integers(cmin, cmax + 1, (5, 256)).astype(np.int8)
    sr = ora.f32_to_bf16(np.exp(rng.uniform(-20, 20, (5, 2))).astype(np.float32))
    w32, _ = ora.dequant(cr, sr)
    assert np.array_equal(ora.requantize(w32, sr, grid), cr)


def test_quantize_rejects_nonfinite(ora):
    W = np.zeros((1, 128), np.float32)
    W[0, 5] = np.nan
    with pytest.raises(ValueError):
        ora.quantize(W, I2)


def test_mixed_rows_follow_their_block(ora):
    W = synth.weight(300, 256, seed=4).numpy()
    table = np.array([I3, T, I2], np.int8)
    c, s = ora.quantize(W, table)
    for b, g in enumerate(table):
        cb, sb = ora.quantize(W[b * 128:(b + 1) * 128], int(g))
        assert np.array_equal(c[b * 128:(b + 1) * 128], cb)
        assert np.array_equal(s[b * 128:(b + 1) * 128], sb)


# ---------------------------------------------------------------- packing
def _packed_row(ora, codes_row, grid):
    """The row's bytes in grid order, read back out of a 1-row packed matrix."""
    K = codes_row.shape[0]
    p = ora.pack(codes_row[None, :].astype(np.int8), grid)
    rb = ora.row_bytes(grid, K)
    # row 0 of slab 0: 16 bytes at chunk*1024
    return np.concatenate([p[c * 1024:c * 1024 + 16] for c in range(rb // 16)])


def _tern_input(j, i):
    """Input index of digit i (weight 3^i) of ternary byte j, layout version 2: even bytes hold
    inputs 5j..5j+4 in digit order; odd bytes hold inputs 5j+1..5j+4 as digits 0..3 and input 5j
    as digit 4 (so the input pairs (10q+6, 10q+7) and (10q+8, 10q+9) are digit pairs (0,1), (2,3))."""
    if j % 2 == 0:
        return 5 * j + i
    return 5 * j + 1 + i if i < 4 else 5 * j


def test_ternary_every_byte_value(ora):
    """All 243 trit tuples <-> byte values 0..242, in even and in odd bytes; byte = the tuple read as
    a base-3 number, digit i taken from input _tern_input(j, i) (Python int(..., 3) as the
    independent decoder)."""
    K = 2560  # 512 bytes, exactly 32 chunks
    for parity in (0, 1):
        codes = np.zeros(K, np.int8)
        js = [2 * v + parity for v in range(243)]
        for v, j in zip(range(243), js):
            digits = np.base_repr(v, 3).zfill(5)[::-1]  # least significant first
            for i in range(5):
                codes[_tern_input(j, i)] = int(digits[i]) - 1
        row = _packed_row(ora, codes, T)
        for v, j in zip(range(243), js):
            digits = "".join(str(codes[_tern_input(j, i)] + 1) for i in range(5))
            assert row[j] == v == int(digits[::-1], 3)
        assert np.array_equal(ora.unpack(ora.pack(codes[None], T), 1, K, T)[0], codes)


def test_ternary_odd_byte_digit_order(ora):
    """A single -1 (digit 0) among 0 codes (digit 1) at each input of a byte pair lands on the
    digit the layout names: byte value 121 - 3^digit."""
    for k in range(10, 20):
        codes = np.zeros(128, np.int8)
        codes[k] = -1
        row = _packed_row(ora, codes, T)
        j = k // 5
        digit = {10: 0, 11: 1, 12: 2, 13: 3, 14: 4, 15: 4, 16: 0, 17: 1, 18: 2, 19: 3}[k]
        assert row[j] == 121 - 3 ** digit, (k, row[j])
        assert all(row[i] == 121 for i in range(26) if i != j)


def test_ternary_rejects_bytes_above_242(ora):
    K = 128
    p = ora.pack(np.zeros((1, K), np.int8), T)
    for bad in (243, 250, 255):
        q = p.copy()
        q[3] = bad
        with pytest.raises(ValueError):
            ora.unpack(q, 1, K, T)


def test_ternary_padding(ora):
    # K=128: 26 bytes of trits (130), two padding trits, padded to 32 bytes; padding code 0 -> digit 1
    assert ora.row_bytes(T, 128) == 32 and ora.row_bytes(T, 4096) == 832 and ora.row_bytes(T, 5120) == 1024
    row = _packed_row(ora, -np.ones(128, np.int8), T)
    assert np.all(row[:25] == 0)
    # byte 25 (odd): digits 0..3 = inputs 126..129 (126, 127 are -1; 128, 129 padding), digit 4 = 125
    assert row[25] == 0 + 0 * 3 + 1 * 9 + 1 * 27 + 0 * 81
    assert np.all(row[26:] == 121)  # five padding digits of 1: 1+3+9+27+81


@pytest.mark.parametrize("pos", range(16))
def test_i2_each_value_each_position(ora, pos):
    for c in range(-2, 2):
        codes = np.full(128, -2, np.int8)  # digit 0 elsewhere
        codes[16 + pos] = c
        row = _packed_row(ora, codes, I2)
        words = row.view("<u4")
        assert words[1] == (c + 2) << (2 * pos)
        assert np.all(np.delete(words, 1) == 0)


# bit positions of code i (0..31) in the 96-bit triple, low bit first: the layout puts code i at
# bits 3i..3i+2 of w0 | w1<<32 | w2<<64 (codes 10 and 21 straddle words)
def _i3_bits(i):
    return [3 * i, 3 * i + 1, 3 * i + 2]


@pytest.mark.parametrize("pos", range(32))
def test_i3_each_value_each_position(ora, pos):
    for c in range(-4, 4):
        codes = np.full(128, -4, np.int8)
        codes[32 * 2 + pos] = c
        row = _packed_row(ora, codes, I3)
        trip = row[24:36]
        big = int.from_bytes(trip.tobytes(), "little")
        want = sum(((c + 4) >> b & 1) << bit for b, bit in enumerate(_i3_bits(pos)))
        assert big == want
        assert np.all(row[:24] == 0) and np.all(row[36:] == 0)


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (64, 384), (129, 640), (200, 4096)])
@pytest.mark.parametrize("grid", [T, I2, I3])
def test_pack_round_trip(ora, N, K, grid):
    rng = np.random.default_rng(N * 7 + K + grid)
    cmin, cmax = GRIDS[grid]
    codes = rng.integers(cmin, cmax + 1, (N, K)).astype(np.int8)
    p = ora.pack(codes, grid)
    assert p.size == ((N + 63) // 64) * 64 * ora.row_bytes(grid, K) or grid is None
    assert np.array_equal(ora.unpack(p, N, K, grid), codes)


def test_slab_interleave_offsets(ora):
    """Row r of slab s, chunk c sits at s*64*row_bytes + c*1024 + r*16 (uniform grid)."""
    N, K = 130, 256
    codes = np.zeros((N, K), np.int8) - 2
    for n in range(N):
        codes[n, 0] = (n % 4) - 2  # word 0 of row n carries its id in the first code
        codes[n, 1] = ((n // 4) % 4) - 2
    p = ora.pack(codes, I2)
    rb = ora.row_bytes(I2, K)
    assert p.size == 3 * 64 * rb
    for n in range(N):
        s, r = divmod(n, 64)
        w = p[s * 64 * rb + r * 16: s * 64 * rb + r * 16 + 4].view("<u4")[0]
        assert w == (n % 4) | (((n // 4) % 4) << 2)


def test_mixed_block_offsets_and_round_trip(ora):
    N, K = 300, 384
    table = np.array([T, I3, I2], np.int8)
    off = ora.block_offsets(N, K, table)
    rb = [ora.row_bytes(g, K) for g in table]
    assert list(off) == [0, 128 * rb[0], 128 * rb[0] + 128 * rb[1], 128 * rb[0] + 128 * rb[1] + 64 * rb[2]]
    rng = np.random.default_rng(1)
    codes = np.concatenate([rng.integers(*GRIDS[int(g)], (min(128, N - b * 128), K), endpoint=True)
                            for b, g in enumerate(table)]).astype(np.int8)
    p = ora.pack(codes, table)
    assert p.size == off[-1]
    assert np.array_equal(ora.unpack(p, N, K, table), codes)


def test_scale_layout(ora):
    N, K = 70, 1280  # G = 10 -> two octets
    rng = np.random.default_rng(2)
    s = rng.integers(0, 2 ** 15, (N, K // 128)).astype(np.uint16)
    ps = ora.pack_scales(s, K)
    assert ps.size == 2 * 2 * 64 * 8
    for n in range(N):
        for g in range(K // 128):
            assert ps[(((n // 64) * 2 + g // 8) * 64 + n % 64) * 8 + g % 8] == s[n, g]
    assert np.array_equal(ora.unpack_scales(ps, N, K), s)


# ---------------------------------------------------------------- dequant
def test_dequant_exact(ora):
    rng = np.random.default_rng(3)
    codes = rng.integers(-4, 4, (4, 256)).astype(np.int8)
    scales = ora.f32_to_bf16(np.exp(rng.uniform(-60, 60, (4, 2))).astype(np.float32))
    w32, w16 = ora.dequant(codes, scales)
    sf = f32_of_bf16(scales)
    for n in range(4):
        for k in range(256):
            assert Fraction(float(w32[n, k])) == int(codes[n, k]) * Fraction(float(sf[n, k // 128]))
    assert np.array_equal(w16, torch_bf16_bits(w32))


# ---------------------------------------------------------------- product
def _exact_sum_check(ora, codes, scales, xbits):
    y = ora.gemv(codes, scales, xbits, threads=1)
    w32, _ = ora.dequant(codes, scales)
    xf = f32_of_bf16(xbits)
    M, K = xf.shape
    N = codes.shape[0]
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(w32[n, k])) * Fraction(float(xf[m, k])) for k in range(K)]
            exact = sum(terms)
            bound = K * 2.0 ** -53 * float(sum(abs(t) for t in terms)) * 1.01
            assert abs(float(Fraction(y[m, n]) - exact)) <= bound


def test_gemv_exact_rational_sum(ora):
    W = synth.weight(5, 256, seed=8).numpy()
    for grid in (T, I2, I3):
        c, s = ora.quantize(W, grid)
        x = synth.bf16_bits(synth.activations(2, 256, seed=9))
        _exact_sum_check(ora, c, s, x)


def test_gemv_matches_float64_matmul(ora):
    W = synth.weight(200, 640, seed=12).numpy()
    table = np.array([I3, T], np.int8)
    c, s = ora.quantize(W, table)
    x = synth.bf16_bits(synth.activations(3, 640, seed=13))
    y = ora.gemv(c, s, x)
    w32, _ = ora.dequant(c, s)
    ref = torch.from_numpy(f32_of_bf16(x).astype(np.float64)) @ torch.from_numpy(w32.astype(np.float64)).T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12 * np.abs(ref.numpy()).max())


def test_gemv_closed_forms(ora):
    K = 512
    one = ora.f32_to_bf16(np.ones(1, np.float32))[0]
    for grid, (cmin, cmax) in GRIDS.items():
        for c in range(cmin, cmax + 1):
            codes = np.full((2, K), c, np.int8)
            scales = np.full((2, K // 128), one, np.uint16)
            x = np.full((1, K), one, np.uint16)
            assert np.all(ora.gemv(codes, scales, x) == c * K)
            # alternating +1/-1 activations cancel exactly
            xa = ora.f32_to_bf16(np.tile([1.0, -1.0], K // 2).astype(np.float32))[None]
            assert np.all(ora.gemv(codes, scales, xa) == 0)


def test_gemv_one_hot_column(ora):
    W = synth.weight(7, 384, seed=14).numpy()
    c, s = ora.quantize(W, I3)
    w32, _ = ora.dequant(c, s)
    one = ora.f32_to_bf16(np.ones(1, np.float32))[0]
    for k in (0, 1, 127, 128, 200, 383):
        x = np.zeros((1, 384), np.uint16)
        x[0, k] = one
        assert np.array_equal(ora.gemv(c, s, x)[0], w32[:, k].astype(np.float64))


def test_gemv_packed_equals_gemv_and_thread_count_free(ora):
    N, K = 300, 1280
    W = synth.weight(N, K, seed=15).numpy()
    table = np.array([T, I2, I3], np.int8)
    c, s = ora.quantize(W, table)
    x = synth.bf16_bits(synth.activations(2, K, seed=16))
    y1 = ora.gemv(c, s, x, threads=1)
    y8 = ora.gemv(c, s, x, threads=8)
    yp = ora.gemv_packed(ora.pack(c, table), ora.pack_scales(s, K), x, N, K, table, threads=3)
    assert np.array_equal(y1, y8) and np.array_equal(y1, yp)


def test_gemv_w16_exact_rational_sum(ora):
    """The bf16-weight product is the fp64 sum of bf16_rne(c*s) * x (w16 itself is pinned
    to torch's bf16 rounding by test_dequant_exact), within the fp64 summation bound."""
    W = synth.weight(4, 256, seed=18).numpy()
    for grid in (T, I2, I3):
        c, s = ora.quantize(W, grid)
        x = synth.bf16_bits(synth.activations(2, 256, seed=19))
        y = ora.gemv_w16(c, s, x, threads=1)
        _, w16 = ora.dequant(c, s)
        wf = f32_of_bf16(w16)
        xf = f32_of_bf16(x)
        for m in range(2):
            for n in range(4):
                terms = [Fraction(float(wf[n, k])) * Fraction(float(xf[m, k])) for k in range(256)]
                bound = 256 * 2.0 ** -53 * float(sum(abs(t) for t in terms)) * 1.01
                assert abs(float(Fraction(y[m, n]) - sum(terms))) <= bound


def test_gemv_w16_differs_only_at_codes_of_magnitude_three(ora):
    """bf16_rne(c*s) == c*s unless |c| = 3 (c*s then needs up to two more significant bits), so
    ternary and 2-bit rows agree bit for bit with gemv, and 3-bit rows do once the codes of
    magnitude 3 are removed; with them the difference stays within 2^-9 of each such term."""
    N, K = 64, 512
    W = synth.weight(N, K, seed=20).numpy()
    x = synth.bf16_bits(synth.activations(3, K, seed=21))
    for grid in (T, I2):
        c, s = ora.quantize(W, grid)
        assert np.array_equal(ora.gemv_w16(c, s, x), ora.gemv(c, s, x))
    c, s = ora.quantize(W, I3)
    assert (np.abs(c) == 3).any()
    c0 = np.where(np.abs(c) == 3, 0, c).astype(np.int8)
    assert np.array_equal(ora.gemv_w16(c0, s, x), ora.gemv(c0, s, x))
    w32, _ = ora.dequant(c, s)
    xf = f32_of_bf16(x).astype(np.float64)
    bound = (np.abs(c) == 3) * np.abs(w32.astype(np.float64)) * 2.0 ** -9
    d = np.abs(ora.gemv_w16(c, s, x) - ora.gemv(c, s, x))
    assert np.all(d <= np.abs(xf) @ bound.T * 1.0001 + 1e-300)
    assert d.max() > 0  # the rounding is real


def test_gemv_w16_one_hot_column(ora):
    W = synth.weight(7, 384, seed=22).numpy()
    c, s = ora.quantize(W, I3)
    _, w16 = ora.dequant(c, s)
    one = ora.f32_to_bf16(np.ones(1, np.float32))[0]
    for k in (0, 5, 127, 128, 300, 383):
        x = np.zeros((1, 384), np.uint16)
        x[0, k] = one
        assert np.array_equal(ora.gemv_w16(c, s, x)[0], f32_of_bf16(w16[:, k]).astype(np.float64))


def test_rel_err_definition(ora):
    y64 = np.array([[3.0, 4.0], [0.0, 1.0]])
    yg = np.array([[3.0, 4.5], [0.0, 1.0]])
    e, nw = ora.rel_err(yg, y64)
    assert e == pytest.approx(0.5 / 5.0) and nw == pytest.approx(0.5 / np.sqrt(26))


# ---------------------------------------------------------------- 4-bit container baseline
# The container is this project's definition of the format the summary page
# (section "Premises & limits") says published checkpoints use: each code as a
# two's complement nibble, the lower input in the low nibble, rows in the same
# 64-row slab interleave as the packed layout.  Pins: literal bytes worked out
# by hand from that definition, positions in the slab interleave, the size
# (4 + 16/128 = 4.125 bits per weight with scales), exhaustive round trips.

def test_c4_hand_computed_bytes(ora):
    codes = np.zeros((1, 128), np.int8)
    codes[0, :8] = [-1, 2, -8, 7, 3, -4, 0, -2]
    b = ora.c4_pack(codes)
    # -1 -> 0xF, 2 -> 0x2 => 0x2F; -8 -> 0x8, 7 -> 0x7 => 0x78; 3, -4 (0xC) => 0xC3; 0, -2 (0xE) => 0xE0
    assert list(b[:4]) == [0x2F, 0x78, 0xC3, 0xE0]
    assert not b[4:].any()


def test_c4_slab_positions(ora):
    N, K = 130, 256
    codes = np.zeros((N, K), np.int8)
    codes[5, 70] = -3     # row 5, byte 35 (high nibble... input 70 is even -> low nibble)
    codes[5, 71] = 1      # same byte, high nibble
    codes[129, 255] = 6   # slab 2, row 1, byte 127 (high nibble)
    b = ora.c4_pack(codes)
    assert len(b) == 3 * 64 * 128 and ora.lib().ora_c4_bytes(N, K) == len(b)
    # byte 35 of row 5: chunk 2 (bytes 32..47), offset 3 -> 2*1024 + 5*16 + 3
    assert b[2 * 1024 + 5 * 16 + 3] == (13 + 16 * 1)
    # slab 2 starts at 2 * 64 * 128; byte 127 of row 1: chunk 7, offset 15
    assert b[2 * 64 * 128 + 7 * 1024 + 1 * 16 + 15] == 6 * 16
    assert np.count_nonzero(b) == 2


def test_c4_bits_per_weight(ora):
    N, K = 4096, 4096
    c4 = ora.lib().ora_c4_bytes(N, K)
    sc = 2 * ora.lib().ora_packed_scales_len(N, K)
    assert (c4 + sc) * 8 / (N * K) == 4.125


@pytest.mark.parametrize("pos", range(32))
def test_c4_every_value_at_every_chunk_position(ora, pos):
    codes = np.zeros((16, 128), np.int8)
    for v in range(-8, 8):
        codes[v + 8, pos] = v
        codes[v + 8, 32 + pos] = -1 - v  # and its complement in the next chunk
    b = ora.c4_pack(codes)
    assert np.array_equal(ora.c4_unpack(b, 16, 128), codes)
    for v in range(-8, 8):
        r = v + 8
        byte = b[(pos // 2) // 16 * 1024 + r * 16 + (pos // 2) % 16]
        nib = (byte >> 4) if pos % 2 else (byte & 15)
        assert nib == (v & 15)


def test_c4_random_round_trip_and_range(ora):
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, (70, 384)).astype(np.int8)
    assert np.array_equal(ora.c4_unpack(ora.c4_pack(codes), 70, 384), codes)
    for bad in (-9, 8):
        c = codes.copy()
        c[3, 7] = bad
        with pytest.raises(ValueError):
            ora.c4_pack(c)
