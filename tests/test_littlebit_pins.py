"""LittleBit oracle pins (CPU): the digest page's bits-per-weight formula and its
two rank examples, the storage count the formula stands for, the forward pass
against a dense reconstruction computed with a library matmul, closed forms,
and hand-placed bits of the packed layout; then the library's host helpers
against the oracle."""
import ctypes

import numpy as np
import pytest

from decode_gemv_thinkbit_amd import qlinear as ql

ONE = np.uint16(0x3F80)


def bf16(a):
    import oracle
    return oracle.f32_to_bf16(np.asarray(a, np.float32))


def test_page_rank_examples(ora):
    # "Rank sets the BPW": a 4096 x 4096 layer at 0.55 BPW needs r = 546, a 4096 x 11008
    # layer at 0.1 BPW needs r = 133
    assert ora.lb_rank(4096, 4096, 0.55) == 546
    assert ora.lb_rank(4096, 11008, 0.1) == 133
    assert ora.lb_rank(11008, 4096, 0.1) == 133
    for (do, di, b) in ((4096, 4096, 0.55), (4096, 11008, 0.1), (28672, 8192, 0.1), (8192, 8192, 1.0)):
        r = ora.lb_rank(do, di, b)
        assert ora.lb_bpw(do, di, r) <= b < ora.lb_bpw(do, di, r + 1)


@pytest.mark.parametrize("do,di,r", [(4096, 4096, 546), (11008, 4096, 133), (300, 128, 7)])
def test_bpw_is_the_storage_of_two_paths(ora, do, di, r):
    # per path: two binary matrices (d_out x r, d_in x r) of 1 bit, three 16-bit scale vectors
    bits = 2 * (r * do + r * di + 16 * (do + di + r))
    assert ora.lb_bpw(do, di, r) == pytest.approx(bits / (do * di), rel=1e-15)


def dense(u, v, g, l, h):
    """W_hat = sum over paths of diag(h) U diag(l) V^T diag(g) (float64, numpy matmul)."""
    f = lambda a: ora_f32(a).astype(np.float64)
    W = 0
    for p in range(2):
        W = W + (f(h[p])[:, None] * (u[p].astype(np.float64) * f(l[p])[None, :])) @ (v[p].astype(np.float64).T * f(g[p])[None, :])
    return W


def ora_f32(bits):
    import oracle
    return oracle.bf16_to_f32(bits)


@pytest.mark.parametrize("do,di,r,seed", [(5, 128, 3, 0), (70, 256, 19, 1), (130, 384, 64, 2), (64, 128, 129, 3)])
def test_forward_equals_dense_reconstruction(ora, do, di, r, seed):
    rng = np.random.default_rng(seed)
    u = rng.choice([-1, 1], (2, do, r)).astype(np.int8)
    v = rng.choice([-1, 1], (2, di, r)).astype(np.int8)
    g, l, h = bf16(rng.uniform(0.5, 2, (2, di))), bf16(rng.uniform(0.1, 1, (2, r))), bf16(rng.uniform(0.01, 0.1, (2, do)))
    x = bf16(rng.standard_normal(di))
    y = ora.lb_gemv(u, v, g, l, h, x)
    y_ref = dense(u, v, g, l, h) @ ora_f32(x).astype(np.float64)
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())


def test_forward_closed_forms(ora):
    do, di, r = 70, 256, 9
    ones = lambda *s: np.full(s, ONE, np.uint16)
    x = bf16(np.linspace(-1, 1, di))
    # all signs +1, unit scales: y_n = 2 paths * r * sum(x)
    y = ora.lb_gemv(np.ones((2, do, r), np.int8), np.ones((2, di, r), np.int8), ones(2, di), ones(2, r), ones(2, do), x)
    assert np.allclose(y, 2 * r * ora_f32(x).astype(np.float64).sum(), rtol=1e-14)
    # path 1 the negation of path 0 (U signs flipped): the paths cancel exactly
    rng = np.random.default_rng(7)
    u0 = rng.choice([-1, 1], (do, r)).astype(np.int8)
    v0 = rng.choice([-1, 1], (di, r)).astype(np.int8)
    y = ora.lb_gemv(np.stack([u0, -u0]), np.stack([v0, v0]), ones(2, di), ones(2, r), ones(2, do), x)
    assert np.all(y == 0.0)


def test_pack_hand_placed_bits(ora):
    do, di, r = 70, 256, 200
    u = np.ones((2, do, r), np.int8)
    v = np.ones((2, di, r), np.int8)
    u[1, 5, 3] = -1    # row 5; path 1's part starts at byte 32 (2 x 16-byte chunks per path); bit 3
    v[1, 130, 7] = -1  # latent row 256 + 7 (path 1 after 256 padded rows), input 130 -> byte 16, bit 2
    ub, vb = ora.lb_pack(u, v)
    assert len(ub) == 2 * 64 * 64 and len(vb) == 2 * 256 * 32
    assert np.count_nonzero(ub) == 1 and ub[2 * 1024 + 5 * 16 + 0] == 1 << 3
    # row 263: slab 4 (rows of 32 bytes), slab row 7; byte 16 = chunk 1, offset 0
    assert np.count_nonzero(vb) == 1 and vb[4 * 64 * 32 + 1 * 1024 + 7 * 16 + 0] == 1 << 2
    u2, v2 = ora.lb_unpack(ub, vb, do, di, r)
    assert np.array_equal(u2, u) and np.array_equal(v2, v)


def test_pack_round_trip_and_rejection(ora):
    rng = np.random.default_rng(9)
    u = rng.choice([-1, 1], (2, 130, 77)).astype(np.int8)
    v = rng.choice([-1, 1], (2, 384, 77)).astype(np.int8)
    ub, vb = ora.lb_pack(u, v)
    u2, v2 = ora.lb_unpack(ub, vb, 130, 384, 77)
    assert np.array_equal(u2, u) and np.array_equal(v2, v)
    u[0, 0, 0] = 0
    with pytest.raises(ValueError):
        ora.lb_pack(u, v)


def test_library_helpers_match_oracle(ora):
    for (do, di, b) in ((4096, 4096, 0.55), (11008, 4096, 0.1), (28672, 8192, 0.1), (28672, 8192, 0.55),
                        (28672, 8192, 1.0), (8192, 8192, 0.1), (1024, 4096, 0.3), (300, 128, 2.0)):
        r = ora.lb_rank(do, di, b)
        assert ql.lb_rank(do, di, b) == r
        assert ql.lb_bpw(do, di, r) == ora.lb_bpw(do, di, r)
        assert ql.lib().qlinear_lb_u_bytes(do, r) == ora.lib().ora_lb_u_bytes(do, r)
        assert ql.lib().qlinear_lb_v_bytes(di, r) == ora.lib().ora_lb_v_bytes(di, r)
        assert ql.lib().qlinear_lb_workspace_bytes(do, di, r) > 0
    assert ql.lib().qlinear_lb_v_bytes(100, 5) == 0 and ql.lib().qlinear_lb_workspace_bytes(64, 100, 5) == 0


def test_lb_argument_errors():
    L = ql.lib()
    p = ctypes.c_void_p(16)
    w = ql.ql_littlebit(64, 128, 5, 0, 16, 16, 16, 16, 16)
    assert L.qlinear_lb_gemv(ctypes.byref(w), p, p, p, 0, None) == 1       # workspace too small
    w.d_in = 100
    assert L.qlinear_lb_gemv(ctypes.byref(w), p, p, p, 1 << 20, None) == 1  # d_in % 128
    w.d_in, w.g = 128, None
    assert L.qlinear_lb_gemv(ctypes.byref(w), p, p, p, 1 << 20, None) == 1  # null scale
    assert L.qlinear_lb_gemv(None, p, p, p, 1 << 20, None) == 1
    assert L.qlinear_lb_pack(64, 128, 0, p, p, p, p, None) == 1              # rank 0
