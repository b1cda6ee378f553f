"""Grouped launches captured in a HIP graph and replayed (needs gfx950).

The per-layer benchmark replays graphs of grouped launches, split and unsplit.
The kernels leave their scheduler and split-K counters at zero themselves (no
memset node), so a graph replays correctly any number of times.  Each replay
here runs after eager work of its own (another grouped launch on the same
stream, a torch op, a synchronization) and must reproduce the eager result bit
for bit (the launches are deterministic), and the counters must be zero after.
"""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu

T, I2, I3 = 0, 1, 2


def note(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def items_for(dev, M, shapes, seed):
    out = []
    for i, (N, K, grid) in enumerate(shapes):
        if grid == "mixed":
            grid = np.array([[I3, T, I2][b % 3] for b in range((N + 127) // 128)], np.int8)
        pw = ql.quantize_pack(synth.weight(N, K, seed=seed + i, device=dev), grid)
        x = synth.activations(M, K, seed=seed + 50 + i, device=dev)
        out.append((pw, x, torch.empty((M, N), device=dev)))
    return out


def zero_state(grp):
    st = grp.sched.cpu().numpy()
    ok = not st[: ql.QL_SCHED_WORDS].any()
    for d in grp.plan:
        if d["kparts"] > 1:
            ok = ok and not st[d["ws_begin"]: d["ws_begin"] + 32 * ((d["N"] + 63) // 64)].any()
    return ok


@pytest.mark.parametrize("M", [1, 4])
def test_graph_replays_of_grouped_launches(dev, M):
    note(f"graph replays M={M}")
    a = items_for(dev, M, [(4096, 4096, "mixed"), (1024, 4096, I3), (1024, 4096, T)], seed=100 + M)
    b = items_for(dev, M, [(4096, 12288, "mixed")], seed=200 + M)
    other = items_for(dev, M, [(512, 1280, I2), (300, 2048, T)], seed=300 + M)
    grps = [ql.GroupedGemv(a, split="auto"), ql.GroupedGemv(b, split="auto"), ql.GroupedGemv(a)]
    assert max(grps[0].kparts) > 1 and max(grps[1].kparts) > 1
    g_other = ql.GroupedGemv(other, split=3)
    # eager reference (a's outputs from the unsplit launch are checked against it too)
    grps[0].run()
    grps[1].run()
    torch.cuda.synchronize()
    ref_a = [y.clone() for _, _, y in a]
    ref_b = [y.clone() for _, _, y in b]
    g_other.run()
    torch.cuda.synchronize()
    ref_o = [y.clone() for _, _, y in other]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grps[0].run()
        grps[1].run()
    for rep in range(4):
        for _, _, y in a + b:
            y.fill_(float("nan"))
        g_other.run()  # eager work of the program between replays, same state-free kernels
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (_, _, y), r in zip(a, ref_a):
            assert torch.equal(y, r), rep
        for (_, _, y), r in zip(b, ref_b):
            assert torch.equal(y, r), rep
        for (_, _, y), r in zip(other, ref_o):
            assert torch.equal(y, r), rep
        assert all(zero_state(g) for g in grps[:2] + [g_other]), rep
    # the unsplit launch of a agrees with the split one within the sum-order bound
    grps[2].run()
    torch.cuda.synchronize()
    for (_, _, y), r in zip(a, ref_a):
        d = (y - r).abs().max().item() / max(r.norm().item() / np.sqrt(r.shape[0]), 1e-30)
        assert d <= 1e-5, d
