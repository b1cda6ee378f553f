"""Property-based GPU parity (needs gfx950): hypothesis draws random shapes, grids (uniform and
per-block tables), batch sizes and K splits (derandomized: every run draws the same cases),
and each case is held to the same bars as the fixed-shape tests: bit-exact codes and
dequantized weights, max_n |dy| / ||y_row||_2 <= 2e-3 (GEMV) / 1e-2 (GEMM) against the
oracle's fp64 product with the normwise tripwires, and the grouped launches against the
oracle entry by entry.
"""
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2
GEMV_TOL, GEMM_TOL, TRIP_GEMV = 2e-3, 1e-2, 1e-5
GPU_PROP = settings(max_examples=25, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


@st.composite
def cases(draw, max_n=700, max_groups=40):
    N = draw(st.integers(1, max_n))
    K = 128 * draw(st.integers(1, max_groups))
    if draw(st.booleans()):
        grid = draw(st.sampled_from([T, I2, I3]))
    else:
        grid = np.array(draw(st.lists(st.sampled_from([T, I2, I3]), min_size=(N + 127) // 128,
                                      max_size=(N + 127) // 128)), np.int8)
    return N, K, grid, draw(st.integers(0, 2**31 - 1))


def make(ora, dev, N, K, grid, seed, M):
    W = synth.weight(N, K, seed=seed)
    c_ref, s_ref = ora.quantize(W.numpy(), grid)
    pw = ql.quantize_pack(W.to(dev), grid)
    x = synth.activations(M, K, seed=seed + 1)
    return pw, x, c_ref, s_ref


@GPU_PROP
@given(cases(), st.integers(1, 16))
def test_prop_gemv(ora, dev, case, M):
    N, K, grid, seed = case
    note(f"prop gemv N={N} K={K} grid={grid if np.isscalar(grid) else 'table'} M={M} seed={seed}")
    pw, x, c_ref, s_ref = make(ora, dev, N, K, grid, seed, M)
    assert np.array_equal(ql.unpack(pw).cpu().numpy(), c_ref)
    y = ql.gemv(x.to(dev), pw).cpu().numpy()
    err, nw = ora.rel_err(y, ora.gemv(c_ref, s_ref, synth.bf16_bits(x)))
    assert err <= GEMV_TOL and nw <= TRIP_GEMV, (err, nw)


@GPU_PROP
@given(cases(max_n=600, max_groups=24), st.integers(1, 300))
def test_prop_gemm(ora, dev, case, M):
    N, K, grid, seed = case
    note(f"prop gemm N={N} K={K} grid={grid if np.isscalar(grid) else 'table'} M={M} seed={seed}")
    pw, x, c_ref, s_ref = make(ora, dev, N, K, grid, seed, M)
    y = ql.gemm(x.to(dev), pw).cpu().numpy()
    xb = synth.bf16_bits(x)
    err, nw = ora.rel_err(y, ora.gemv(c_ref, s_ref, xb))
    assert N < 64 or err <= GEMM_TOL, (err, nw)
    ref = ora.gemv_w16(c_ref, s_ref, xb) if M >= 16 else ora.gemv(c_ref, s_ref, xb)
    _, nw2 = ora.rel_err(y, ref)
    assert nw2 <= (TRIP_GEMV if M >= 16 else 1e-4), nw2


@GPU_PROP
@given(st.lists(cases(max_n=400, max_groups=30), min_size=1, max_size=5), st.integers(1, 16),
       st.sampled_from([None, "auto", 2, 5]))
def test_prop_grouped_gemv(ora, dev, items, M, split):
    note(f"prop grouped gemv {[(n, k) for n, k, _, _ in items]} M={M} split={split}")
    made = [make(ora, dev, N, K, grid, seed, M) for N, K, grid, seed in items]
    ys = [torch.empty((M, pw.N), device=dev) for pw, _, _, _ in made]
    ql.GroupedGemv([(pw, x.to(dev), y) for (pw, x, _, _), y in zip(made, ys)], split=split).run()
    torch.cuda.synchronize()
    for (pw, x, c_ref, s_ref), y in zip(made, ys):
        err, nw = ora.rel_err(y.cpu().numpy(), ora.gemv(c_ref, s_ref, synth.bf16_bits(x)))
        assert err <= GEMV_TOL and nw <= TRIP_GEMV, (pw.N, pw.K, err, nw)


@GPU_PROP
@given(st.lists(cases(max_n=400, max_groups=24), min_size=1, max_size=5), st.integers(16, 300))
def test_prop_grouped_gemm(ora, dev, items, M):
    note(f"prop grouped gemm {[(n, k) for n, k, _, _ in items]} M={M}")
    made = [make(ora, dev, N, K, grid, seed, M) for N, K, grid, seed in items]
    ys = [torch.empty((M, pw.N), device=dev) for pw, _, _, _ in made]
    ql.GroupedGemm([(pw, x.to(dev), y) for (pw, x, _, _), y in zip(made, ys)]).run()
    torch.cuda.synchronize()
    for (pw, x, c_ref, s_ref), y in zip(made, ys):
        xb = synth.bf16_bits(x)
        yy = y.cpu().numpy()
        err, _ = ora.rel_err(yy, ora.gemv(c_ref, s_ref, xb))
        assert pw.N < 64 or err <= GEMM_TOL, (pw.N, pw.K, err)
        _, nw16 = ora.rel_err(yy, ora.gemv_w16(c_ref, s_ref, xb))
        assert nw16 <= TRIP_GEMV, (pw.N, pw.K, nw16)
