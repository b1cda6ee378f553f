"""qlinear_gemv_grouped_noalloc (state in the library's static device array) against
qlinear_gemv_grouped (state in a caller buffer), needs gfx950.

Both run the same kernels on the same descriptor lists, so their outputs must be
bitwise equal; each is also held to the oracle's GEMV bar.  Two calls in a row,
the second with a smaller input (fewer, shorter rows, another batch size), and a
third back at the first shape, check that the array's reuse (counters left at
zero, stale partial sums from the larger call) changes nothing.
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


def mixed(N, seed):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, 3, (N + 127) // 128).astype(np.int8)
    t[0] = 2
    return t


def build(ora, dev, cases, M, seed0):
    items, refs = [], []
    for i, (N, K, grid) in enumerate(cases):
        g = mixed(N, seed0 + i) if grid == "mixed" else grid
        W = synth.weight(N, K, seed=seed0 + i)
        c, s = ora.quantize(W.numpy(), g)
        x = synth.activations(M, K, seed=seed0 + 100 + i)
        refs.append(ora.gemv(c, s, synth.bf16_bits(x)))
        items.append((ql.quantize_pack(W.to(dev), g), x.to(dev)))
    return items, refs


def run_both(items, M, split, dev):
    ys_ref = [torch.full((M, pw.N), float("nan"), device=dev) for pw, _ in items]
    ys = [torch.full((M, pw.N), float("nan"), device=dev) for pw, _ in items]
    g_ref = ql.GroupedGemv([(pw, x, y) for (pw, x), y in zip(items, ys_ref)], split=split)
    g_na = ql.GroupedGemv([(pw, x, y) for (pw, x), y in zip(items, ys)], split=split, noalloc=True)
    assert g_na.sched is None and g_na.state_words == g_ref.state_words
    g_ref.run()
    g_na.run()
    torch.cuda.synchronize()
    return ys_ref, ys


def check(ora, ys_ref, ys, refs, what):
    for y_ref, y, y64 in zip(ys_ref, ys, refs):
        assert torch.equal(y, y_ref), what
        err, nw = ora.rel_err(y.cpu().numpy(), y64)
        assert err <= 2e-3 and nw <= 1e-5, (what, err, nw)


def test_noalloc_matches_caller_state_two_calls(ora, dev):
    big = [(4096, 4096, "mixed"), (1024, 4096, I3), (12288, 4096, T), (4096, 12288, "mixed")]
    small = [(300, 1280, T), (129, 640, I2), (64, 384, "mixed")]
    items_b, refs_b = build(ora, dev, big, 1, 700)
    note("noalloc: first call, M=1, split auto")
    ys_ref, ys = run_both(items_b, 1, "auto", dev)
    check(ora, ys_ref, ys, refs_b, "first call")
    items_s, refs_s = build(ora, dev, small, 4, 800)
    note("noalloc: second call, smaller input, M=4, split 2")
    ys_ref, ys = run_both(items_s, 4, 2, dev)
    check(ora, ys_ref, ys, refs_s, "second call")
    note("noalloc: third call, M=1, no split")
    ys_ref, ys = run_both(items_b, 1, None, dev)
    check(ora, ys_ref, ys, refs_b, "third call")


def test_noalloc_rejects_oversized_state(dev):
    """A launch needing more state than the static array holds is refused before any launch."""
    W = synth.weight(128, 1280, seed=5, device=dev)
    pw = ql.quantize_pack(W, T)
    x = synth.activations(1, 1280, seed=6, device=dev)
    y = torch.empty((1, 128), device=dev)
    g = ql.GroupedGemv([(pw, x, y)])
    st = ql.lib().qlinear_gemv_grouped_noalloc(ql._ptr(g.descs), g.count, g.total, 1,
                                               ql.QL_NOALLOC_STATE_WORDS + 1, ql._stream())
    assert st == 1  # QL_EINVAL
    assert b"static array" in ql.lib().qlinear_last_error()
