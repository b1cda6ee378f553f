"""GPU side of the grid allocation (needs gfx950).

qlinear_rtn_noise against the oracle's rounding noise (fp64 sums in different
orders: relative 1e-12), and the whole allocation of a Qwen3-1.7B layer --
GPU noise, sensitivities, the library's knapsack -- against the oracle's own
pipeline (CPU noise, CPU sensitivities, the oracle's knapsack): the same grid
for every block and every linear.  The allocated tables then drive a grouped
GEMV that must meet the usual contract.
"""
import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import allocation, configs
from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("N,K", [(1, 128), (130, 256), (200, 2048), (1000, 4096), (70, 384), (2048, 6144)])
def test_rtn_noise_matches_oracle(ora, dev, N, K):
    print(f"rtn_noise N={N} K={K}", flush=True)
    W = synth.weight(N, K, seed=900 + N + K)
    if N > 100:
        W[100:110] = 0.0  # all-zero groups: s = 0
    E = ql.rtn_noise(W.to(dev)).cpu().numpy()
    E_ref = ora.rtn_noise(W.numpy())
    assert E.shape == E_ref.shape
    np.testing.assert_allclose(E, E_ref, rtol=1e-12, atol=0)
    # deterministic: a second launch gives the same bits
    assert np.array_equal(ql.rtn_noise(W.to(dev)).cpu().numpy(), E)


@pytest.mark.parametrize("N,K", [(1, 128), (130, 256), (200, 2048), (1024, 17408), (70, 384)])
def test_block_sensitivity_matches_oracle(ora, dev, N, K):
    """qlinear_block_sensitivity against the oracle: bit-exact (ascending fp64 sums on both sides)."""
    x = synth.activations(1, K, seed=N + K).view(-1)
    g = torch.randn(N, generator=torch.Generator().manual_seed(K)) * 3.0
    S = ql.block_sensitivity(x.to(dev), g.to(dev)).cpu().numpy()
    S_ref = ora.block_sensitivity(synth.bf16_bits(x), g.numpy())
    assert np.array_equal(S, S_ref)


def oracle_units(ora, wl, wi, layer, granularity, dev):
    """The oracle's units from the same seeded inputs (drawn on the device, as the
    library's pipeline draws them, and copied to the host)."""
    keys, n, S, E, allowed = [], [], [], [], []
    for mi, lin in enumerate(wl.linears):
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, layer, mi), device=dev).cpu().numpy()
        noise = ora.rtn_noise(W)
        x = synth.bf16_bits(synth.activations(1, lin.K, synth.x_seed(wi, layer, lin.x_slot, 1), device=dev))
        g = synth.output_gradient(lin.N, wi, layer, mi, device=dev).cpu().numpy()
        sb = ora.block_sensitivity(x, g)
        rows = np.minimum(128, lin.N - 128 * np.arange(len(sb)))
        mask = 6 if lin.name in ("q", "k") else 7
        if granularity == "block":
            for b in range(len(sb)):
                keys.append((layer, lin.name, b, 1))
                n.append(int(rows[b]) * lin.K)
                S.append(sb[b])
                E.append(noise[b])
                allowed.append(mask)
        else:
            keys.append((layer, lin.name, 0, len(sb)))
            n.append(lin.N * lin.K)
            S.append(sb.sum())
            E.append(noise.sum(axis=0))
            allowed.append(mask)
    return keys, np.array(n), np.array(S), np.array(E), np.array(allowed, np.uint32)


@pytest.mark.parametrize("granularity", ["block", "linear"])
def test_qwen3_1p7b_layer_allocation_matches_oracle(ora, dev, granularity):
    wl = configs.WORKLOADS["qwen3_1p7b_layer"]
    wi = list(configs.WORKLOADS).index(wl.name)
    tables, (units, grids, lam) = allocation.knapsack_allocation(wl, wi, dev, 2.0, granularity=granularity)
    keys, n, S, E, allowed = oracle_units(ora, wl, wi, 0, granularity, dev)
    assert units.keys == keys and np.array_equal(units.weights, n)
    np.testing.assert_allclose(units.noise, E, rtol=1e-12)
    assert np.array_equal(units.sensitivity, S)  # same sums, same order: bit-exact
    g_ref, lam_ref = ora.allocate(n, S, E, allowed, 2.0)
    assert np.array_equal(grids, g_ref)
    # the library's multiplier sits inside the interval the oracle's assignment holds on
    assert lam >= lam_ref * (1 - 1e-9)
    sh = allocation.shares(units, grids)
    bits = sum(sh[g] * ora.GRID_BITS[g] for g in range(3))
    print(f"{granularity}: shares T {sh[0]:.3f} I2 {sh[1]:.3f} I3 {sh[2]:.3f}, {bits:.4f} bits/weight", flush=True)
    assert bits <= 2.0 + 1e-12
    for name in ("q", "k"):
        assert (tables[0][name] != 0).all()  # q and k keep >= 2 bits


def test_allocated_layer_runs_grouped_gemv(ora, dev):
    """The allocator's tables drive quantize/pack and a grouped GEMV of the layer."""
    wl = configs.WORKLOADS["qwen3_1p7b_layer"]
    wi = list(configs.WORKLOADS).index(wl.name)
    tables, _ = allocation.knapsack_allocation(wl, wi, dev, 2.0)
    items, refs = [], []
    for mi, lin in enumerate(wl.linears):
        W = synth.weight(lin.N, lin.K, synth.weight_seed(wi, 0, mi), device=dev)
        x = synth.activations(1, lin.K, synth.x_seed(wi, 0, lin.x_slot, 1), device=dev)
        c, s = ora.quantize(W.cpu().numpy(), tables[0][lin.name])
        refs.append(ora.gemv(c, s, synth.bf16_bits(x)))
        pw = ql.quantize_pack(W, tables[0][lin.name])
        items.append((pw, x, torch.empty((1, lin.N), device=dev)))
    ql.GroupedGemv(items).run()
    torch.cuda.synchronize()
    for (_, _, y), y64 in zip(items, refs):
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= 2e-3 and nw <= 1e-5, (err, nw)
