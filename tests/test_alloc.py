"""Grid allocation (summary page, section "How it differs", stage 1), on the CPU.

The oracle's pieces are pinned against what the mathematics fixes:
  * the knapsack: brute force over every assignment of tiny instances -- the
    Lagrangian answer must fit the budget, be optimal among all assignments
    using no more bits than it does, and its dual value must bound the true
    optimum from below; closed forms (no sensitivity, unlimited budget);
  * rounding noise: the squared error of the (separately pinned) quantizer's
    codes and scales; zero for weights already on the grid;
  * sensitivity: closed forms.
The oracle solves the knapsack as a greedy walk along each unit's lower convex
hull; the library sweeps the multiplier over its crossing points.  The two are
different computations of the same Lagrangian answer: the brute-force pins run
against both solvers, and the library must pick the oracle's grids exactly.
"""
import itertools

import numpy as np
import pytest

from decode_gemv_thinkbit_amd import qlinear as ql

BITS = np.array([np.log2(3.0) + 1 / 8, 2 + 1 / 8, 3 + 1 / 8])


def random_instance(rng, m, masks=(7, 7, 7, 6, 3, 5)):
    n = rng.integers(1, 50, m) * 128
    S = rng.lognormal(0.0, 1.0, m)
    # noise falls with more bits, as for round-to-nearest
    E = np.sort(rng.uniform(0.01, 1.0, (m, 3)), axis=1)[:, ::-1] * n[:, None]
    allowed = rng.choice(masks, m).astype(np.uint32)
    return n, S, E, allowed


def brute(n, S, E, allowed, cap):
    """(min cost, bits) over every assignment with total bits <= cap."""
    best = (np.inf, None)
    opts = [[g for g in range(3) if allowed[i] >> g & 1] for i in range(len(n))]
    for choice in itertools.product(*opts):
        bits = sum(n[i] * BITS[g] for i, g in enumerate(choice))
        if bits <= cap:
            cost = sum(S[i] * E[i, g] for i, g in enumerate(choice))
            if cost < best[0]:
                best = (cost, bits)
    return best


def test_page_shares_fit_the_two_bit_budget():
    """Reading of the budget: ternary at log2(3) bits plus a bf16 scale per 128 weights.
    The page's 1.7B allocation (75.3 % T, 6.0 % I2, 18.7 % I3) then averages 1.9995 bits,
    inside the 2.0-bit budget it was solved for; with 1.6-bit ternary it would not fit."""
    assert 0.753 * BITS[0] + 0.06 * BITS[1] + 0.187 * BITS[2] == pytest.approx(1.99948, abs=1e-5)
    assert 0.753 * (1.6 + 1 / 8) + 0.06 * BITS[1] + 0.187 * BITS[2] > 2.0


def solve(which, ora, n, S, E, allowed, budget, bits=None):
    """(grids, multiplier) from the oracle or the library; ValueError when infeasible."""
    if which == "oracle":
        return ora.allocate(n, S, E, allowed, budget, bits)
    try:
        return ql.allocate(n, S, E, allowed, budget, bits)
    except ql.QLinearError as e:
        raise ValueError(str(e)) from e


@pytest.mark.parametrize("which", ["oracle", "library"])
@pytest.mark.parametrize("seed", range(40))
def test_knapsack_against_brute_force(ora, seed, which):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(1, 8))
    n, S, E, allowed = random_instance(rng, m)
    budget = float(rng.uniform(1.75, 3.1))
    cap = budget * n.sum()
    cheapest = sum(n[i] * min(BITS[g] for g in range(3) if allowed[i] >> g & 1) for i in range(m))
    if cheapest > cap:
        with pytest.raises(ValueError):
            solve(which, ora, n, S, E, allowed, budget)
        return
    g, lam = solve(which, ora, n, S, E, allowed, budget)
    assert all(allowed[i] >> g[i] & 1 for i in range(m))
    used = float((n * BITS[g]).sum())
    cost = float((S * E[np.arange(m), g]).sum())
    assert used <= cap * (1 + 1e-12)
    # optimal for the bits it uses (the Lagrangian sufficiency theorem)
    opt_own, _ = brute(n, S, E, allowed, used * (1 + 1e-12))
    assert cost <= opt_own * (1 + 1e-12) + 1e-12
    # the dual value bounds the optimum at the full budget from below
    opt_full, _ = brute(n, S, E, allowed, cap)
    dual = sum(min(S[i] * E[i, h] + lam * n[i] * BITS[h] for h in range(3) if allowed[i] >> h & 1)
               for i in range(m)) - lam * cap
    assert dual <= opt_full * (1 + 1e-12) + 1e-12
    assert opt_full <= cost * (1 + 1e-12) + 1e-12


def test_knapsack_duality_gap_example(ora):
    """Three equal units at a budget where two of them could take 2-bit: the exact optimum
    upgrades two, but the three T -> I2 hull edges have one slope, so no multiplier takes
    only two of them and the relaxation leaves all three ternary (the method's known gap)."""
    n = np.array([128, 128, 128])
    S = np.ones(3)
    E = np.array([[10.0, 2.0, 0.0]] * 3) * 128
    budget = (2 * BITS[1] + BITS[0]) / 3 * (1 + 1e-12)
    for which in ("oracle", "library"):
        g, _ = solve(which, ora, n, S, E, np.full(3, 7, np.uint32), budget)
        assert list(g) == [0, 0, 0], (which, g)
    opt, _ = brute(n, S, E, np.full(3, 7), budget * n.sum())
    assert opt == pytest.approx((2.0 + 2.0 + 10.0) * 128)


def test_oracle_knapsack_closed_forms(ora):
    rng = np.random.default_rng(3)
    n, S, E, allowed = random_instance(rng, 30)
    # no sensitivity: every unit takes its cheapest allowed grid, multiplier 0
    g, lam = ora.allocate(n, np.zeros(30), E, allowed, 2.0)
    low = [min((BITS[h], h) for h in range(3) if allowed[i] >> h & 1)[1] for i in range(30)]
    assert list(g) == low and lam == 0.0
    # budget above every grid: the least-noise allowed grid everywhere, multiplier 0
    g, lam = ora.allocate(n, S, E, allowed, 4.0)
    best = [min((E[i, h], h) for h in range(3) if allowed[i] >> h & 1)[1] for i in range(30)]
    assert list(g) == best and lam == 0.0
    # an infeasible budget is rejected
    with pytest.raises(ValueError):
        ora.allocate(n, S, E, np.full(30, 4, np.uint32), 2.0)


def test_oracle_rtn_noise(ora):
    rng = np.random.default_rng(4)
    W = rng.normal(0, 0.02, (200, 384)).astype(np.float32)
    W[130:140] = 0.0
    E = ora.rtn_noise(W)
    assert E.shape == (2, 3)
    for grid in range(3):
        c, s = ora.quantize(W, grid)
        w = c.astype(np.float64) * np.repeat(ora.bf16_to_f32(s).astype(np.float64), 128, axis=1)
        d = (W.astype(np.float64) - w) ** 2
        assert E[0, grid] == pytest.approx(d[:128].sum(), rel=1e-12)
        assert E[1, grid] == pytest.approx(d[128:].sum(), rel=1e-12)
    assert E[0, 0] > E[0, 1] > E[0, 2] > 0
    # weights already on the grid (c * s with s a power of two) have no noise
    c = rng.integers(-4, 4, (64, 256)).astype(np.float32)
    c[:, ::128] = -4  # every group's max |c| is 4, so s = 1/8 * 4 / 4 ... reproduces the codes
    assert ora.rtn_noise(c * 0.125)[0, 2] == 0.0


def test_oracle_block_sensitivity(ora):
    x = np.full(512, 0x4000, np.uint16)  # bf16 2.0 -> ||x||^2 = 2048
    g = np.arange(1, 201, dtype=np.float32)
    S = ora.block_sensitivity(x, g)
    assert S[0] == 2048.0 * sum(i * i for i in range(1, 129))
    assert S[1] == 2048.0 * sum(i * i for i in range(129, 201))


def lagrangian_minimiser(n, S, E, allowed, lam, bits):
    """Per unit, the allowed grid minimising S*E + lam*n*bits, ties to fewer bits."""
    out = []
    for i in range(len(n)):
        opts = sorted((h for h in range(3) if allowed[i] >> h & 1), key=lambda h: (bits[h], h))
        costs = [S[i] * E[i, h] + lam * (n[i] * bits[h]) for h in opts]
        out.append(opts[int(np.argmin(costs))])
    return np.array(out)


@pytest.mark.parametrize("seed", range(20))
def test_library_allocator_matches_oracle(ora, seed):
    """Same grids as the oracle's hull walk; the library's multiplier lies at or above the
    oracle's (the slope of the first group left out) and its Lagrangian minimiser is that
    same assignment."""
    rng = np.random.default_rng(100 + seed)
    m = int(rng.integers(1, 400))
    n, S, E, allowed = random_instance(rng, m, masks=(7, 6, 3, 5, 1, 2, 4))
    if seed % 4 == 0:
        S[rng.integers(0, m, m // 3)] = 0.0
    cases = [(b, None) for b in (1.75, 2.0, 2.4, 3.0)] + [(2.5, np.array([1.6 + 1 / 8, 2.125, 3.125]))]
    for budget, bits in cases:
        try:
            g2, l2 = ora.allocate(n, S, E, allowed, budget, bits)
        except ValueError:
            with pytest.raises(ql.QLinearError):
                ql.allocate(n, S, E, allowed, budget, bits)
            continue
        g1, l1 = ql.allocate(n, S, E, allowed, budget, bits)
        assert np.array_equal(g1, g2), (budget, np.flatnonzero(g1 != g2)[:5])
        assert l1 >= l2
        assert np.array_equal(lagrangian_minimiser(n, S, E, allowed, l1, BITS if bits is None else bits), g1)


def test_allocate_argument_errors():
    n, S, E = [128], [1.0], [[3.0, 2.0, 1.0]]
    with pytest.raises(ql.QLinearError):
        ql.allocate(n, S, E, [0], 2.0)          # no allowed grid
    with pytest.raises(ql.QLinearError):
        ql.allocate(n, S, E, [8], 2.0)          # unknown grid bit
    with pytest.raises(ql.QLinearError):
        ql.allocate(n, [-1.0], E, [7], 2.0)     # negative sensitivity
    with pytest.raises(ql.QLinearError):
        ql.allocate(n, S, [[1.0, np.nan, 0.0]], [7], 2.0)
    with pytest.raises(ql.QLinearError):
        ql.allocate(n, S, E, [4], 2.0)          # 3-bit only cannot fit 2 bits
    with pytest.raises(ql.QLinearError):
        ql.allocate([0], S, E, [7], 2.0)
    assert ql.allocate(n, S, E, [7], 2.0)[0][0] == 0  # one unit, only ternary fits
