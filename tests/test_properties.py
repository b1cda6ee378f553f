"""Property-based checks of the oracle (CPU): random shapes, grids, codes and weights drawn by
hypothesis (derandomized, so every run draws the same examples), each held to a property the
pages or the arithmetic fix rather than to a stored value.

- Layout: pack -> unpack returns the codes (every grid, mixed blocks, ragged rows and
  ternary tails); the packed size is 64 rows' bytes per slab at the slab's grid; the
  slab-packed scales and the 4-bit containers round-trip.
- Quantizer (summary page, "How it works": codes on the grid, one bf16 scale per 128 inputs):
  codes stay on their grid, |w - c s| <= s / 2 for weights inside the grid's range, the
  scale is bf16(max|w| / |c_min|), re-rounding with the stored scales gives the codes back,
  and on small groups it agrees with the brute-force argmin in exact rationals.
- Dequant: w = c * s exactly in fp32.
- Product: the fp64 product is within the gamma_K bound of the exact rational sum.
"""
import importlib.util
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

T, I2, I3 = 0, 1, 2
GRIDS = {T: (-1, 1), I2: (-2, 1), I3: (-4, 3)}

_spec = importlib.util.spec_from_file_location("oracle_pins", os.path.join(os.path.dirname(__file__), "test_oracle_pins.py"))
_pins = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_pins)

PROP = settings(max_examples=40, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


@st.composite
def layouts(draw, max_n=300, max_groups=12):
    """(N, K, grid): an int grid or a per-128-row-block table over all three grids."""
    N = draw(st.integers(1, max_n))
    K = 128 * draw(st.integers(1, max_groups))
    if draw(st.booleans()):
        grid = draw(st.sampled_from([T, I2, I3]))
    else:
        grid = np.array(draw(st.lists(st.sampled_from([T, I2, I3]), min_size=(N + 127) // 128,
                                      max_size=(N + 127) // 128)), np.int8)
    return N, K, grid


def row_grids(N, grid):
    return np.full(N, grid, np.int8) if np.isscalar(grid) or isinstance(grid, int) else np.repeat(grid, 128)[:N]


def random_codes(rng, N, grid):
    g = row_grids(N, grid)
    lo = np.array([GRIDS[int(v)][0] for v in g])[:, None]
    hi = np.array([GRIDS[int(v)][1] for v in g])[:, None]
    return lo, hi, g


@PROP
@given(layouts(), st.integers(0, 2**32 - 1))
def test_prop_pack_round_trip(ora, lay, seed):
    N, K, grid = lay
    rng = np.random.default_rng(seed)
    lo, hi, g = random_codes(rng, N, grid)
    codes = (lo + np.floor(rng.random((N, K)) * (hi - lo + 1))).astype(np.int8)
    packed = ora.pack(codes, grid)
    # every 64-row slab is stored whole (padding rows code zero)
    slab_grids = g[::64]
    assert packed.size == sum(64 * ora.row_bytes(int(v), K) for v in slab_grids)
    assert np.array_equal(ora.unpack(packed, N, K, grid), codes)


@PROP
@given(st.integers(1, 200), st.integers(1, 20), st.integers(0, 2**32 - 1))
def test_prop_scales_and_containers_round_trip(ora, N, groups, seed):
    K = 128 * groups
    rng = np.random.default_rng(seed)
    scales = (rng.integers(0, 0x7F80, (N, groups))).astype(np.uint16)  # finite non-negative bf16
    assert np.array_equal(ora.unpack_scales(ora.pack_scales(scales, K), N, K), scales)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    assert np.array_equal(ora.c4_unpack(ora.c4_pack(codes), N, K), codes)


@st.composite
def weights(draw, max_n=4, max_groups=3):
    N = draw(st.integers(1, max_n))
    G = draw(st.integers(1, max_groups))
    seed = draw(st.integers(0, 2**32 - 1))
    rng = np.random.default_rng(seed)
    kind = draw(st.sampled_from(["normal", "wide", "ties", "zero_groups"]))
    W = (rng.standard_normal((N, 128 * G)) * 0.02).astype(np.float32)
    if kind == "wide":
        W *= np.float32(10.0) ** rng.integers(-30, 30, (N, 1)).astype(np.float32)
    elif kind == "ties":  # exact half-integer multiples of a bf16-exact scale
        s = np.float32(2.0) ** rng.integers(-12, 2)
        W = (rng.integers(-9, 10, W.shape) * np.float32(0.5) * s).astype(np.float32)
    elif kind == "zero_groups":
        W[:, :128] = 0
    return W


@PROP
@given(weights(), st.sampled_from([T, I2, I3]))
def test_prop_quantizer(ora, W, grid):
    cmin, cmax = GRIDS[grid]
    codes, scales = ora.quantize(W, grid)
    N, K = W.shape
    assert codes.min() >= cmin and codes.max() <= cmax
    sf = ora.bf16_to_f32(scales).astype(np.float64)
    for n in range(N):
        for g in range(K // 128):
            w = W[n, 128 * g:128 * (g + 1)].astype(np.float64)
            a = np.float32(np.max(np.abs(W[n, 128 * g:128 * (g + 1)])))
            assert scales[n, g] == ora.f32_to_bf16(np.array([a / np.float32(-cmin)], np.float32))[0]
            s = sf[n, g]
            c = codes[n, 128 * g:128 * (g + 1)].astype(np.float64)
            inside = (w >= cmin * s) & (w <= cmax * s)
            assert np.all(np.abs(w - c * s)[inside] <= s / 2)
            if s == 0:
                assert not c.any()
    assert np.array_equal(ora.requantize(W, scales, grid), codes)
    if N * K <= 512:
        cb, sb = _pins.brute_force_quantize(W, grid)
        assert np.array_equal(cb, codes) and np.array_equal(sb, scales)
    w32, _ = ora.dequant(codes, scales)
    assert np.array_equal(w32.astype(np.float64), codes.astype(np.float64) * np.repeat(sf, 128, axis=1))


@PROP
@given(st.integers(1, 6), st.integers(1, 2), st.integers(1, 3), st.sampled_from([T, I2, I3]),
       st.integers(0, 2**32 - 1))
def test_prop_product_within_bound(ora, N, groups, M, grid, seed):
    K = 128 * groups
    rng = np.random.default_rng(seed)
    cmin, cmax = GRIDS[grid]
    codes = rng.integers(cmin, cmax + 1, (N, K)).astype(np.int8)
    scales = rng.integers(0x3800, 0x4000, (N, groups)).astype(np.uint16)
    x = rng.integers(0x3000, 0x4100, (M, K)).astype(np.uint16) | (rng.integers(0, 2, (M, K)) << 15).astype(np.uint16)
    y = ora.gemv(codes, scales, x)
    w32, _ = ora.dequant(codes, scales)
    xf = ora.bf16_to_f32(x)
    u = 2.0 ** -53
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(w32[n, k])) * Fraction(float(xf[m, k])) for k in range(K)]
            exact = sum(terms)
            bound = K * u / (1 - K * u) * float(sum(abs(t) for t in terms))
            assert abs(float(Fraction(y[m, n]) - exact)) <= bound
