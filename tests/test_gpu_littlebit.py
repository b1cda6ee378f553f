"""GPU parity of the LittleBit GEMV (needs gfx950): packed sign buffers
bit-exact against the oracle's packer; products against the oracle's fp64
forward pass within the GEMV contract (max_n |dy| / ||y||_2 <= 2e-3, normwise
tripwire 1e-5), at small ragged shapes and at the digest page's shapes (every
row); an exact integer case; and determinism."""
import sys

import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql
from decode_gemv_thinkbit_amd import synth

pytestmark = pytest.mark.gpu
TOL, TRIP = 2e-3, 1e-5


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ql.lib()
    return torch.device("cuda:0")


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_case(ora, dev, do, di, r, seed):
    print(f"littlebit d_out={do} d_in={di} r={r}", flush=True)
    sys.stdout.flush()
    u, v, g, l, h = synth.littlebit_params(do, di, r, seed, device=dev)
    lw = ql.lb_pack(u, v, g, l, h)
    x = synth.activations(1, di, seed + 1, device=dev).view(-1)
    y = ql.lb_gemv(x, lw)
    torch.cuda.synchronize()
    un, vn = u.cpu().numpy(), v.cpu().numpy()
    ub, vb = ora.lb_pack(un, vn)
    assert np.array_equal(lw.u_bits.cpu().numpy(), ub)
    assert np.array_equal(lw.v_bits.cpu().numpy(), vb)
    y64 = ora.lb_gemv(un, vn, bits(g), bits(l), bits(h), bits(x))
    err, nw = ora.rel_err(y.cpu().numpy(), y64)
    assert err <= TOL and nw <= TRIP, (err, nw)
    return lw, x, y


@pytest.mark.parametrize("do,di,r", [(1, 128, 1), (70, 256, 19), (130, 384, 64), (64, 128, 129), (200, 2048, 300),
                                     (1000, 4096, 33), (3, 8192, 65)])
def test_littlebit_small_shapes(ora, dev, do, di, r):
    """Inputs of up to 64 chunks of 128 (d_in <= 8192): one workgroup per latent slab."""
    run_case(ora, dev, do, di, r, seed=do + di + r)


@pytest.mark.parametrize("do,di,r", [(300, 8320, 40), (130, 16384, 70), (64, 28672, 129), (257, 12288, 1)])
def test_littlebit_split_latent_shapes(ora, dev, do, di, r):
    """Inputs past 64 chunks of 128: the latent step splits each slab's inputs over waves of
    several workgroups and sums the slices through device memory."""
    run_case(ora, dev, do, di, r, seed=do + di + r)


@pytest.mark.parametrize("do,di,bpw", [(28672, 8192, 0.1), (28672, 8192, 0.55), (11008, 4096, 0.1),
                                       (8192, 8192, 0.1), (11008, 4096, 1.0)])
def test_littlebit_page_shapes_every_row(ora, dev, do, di, bpw):
    """The digest page's kernel shapes (Llama2-70B MLP and attention, Llama2-7B MLP)."""
    run_case(ora, dev, do, di, ql.lb_rank(do, di, bpw), seed=11)


def test_littlebit_exact_integer_case(ora, dev):
    """Unit scales and x = e_i: y_n = sum over paths and latents of U(n, j) V(i, j), an integer."""
    do, di, r = 130, 256, 77
    u, v, _, _, _ = synth.littlebit_params(do, di, r, 5, device=dev)
    one = lambda *s: torch.ones(s, dtype=torch.bfloat16, device=dev)
    lw = ql.lb_pack(u, v, one(2, di), one(2, r), one(2, do))
    un, vn = u.cpu().numpy().astype(np.int64), v.cpu().numpy().astype(np.int64)
    for i in (0, 1, 127, 128, 255):
        x = torch.zeros(di, dtype=torch.bfloat16, device=dev)
        x[i] = 1.0
        y = ql.lb_gemv(x, lw).cpu().numpy()
        ref = (un[0] @ vn[0, i] + un[1] @ vn[1, i]).astype(np.float32)
        assert np.array_equal(y, ref), i


def test_littlebit_deterministic(ora, dev):
    lw, x, y = run_case(ora, dev, 1000, 4096, 150, seed=3)
    for _ in range(3):
        assert torch.equal(ql.lb_gemv(x, lw), y)


@pytest.mark.parametrize("do,di,bpw", [(28672, 8192, 0.1), (1000, 4096, 0.55), (130, 256, 1.0), (200, 16384, 0.3)])
def test_littlebit_reused_workspace(ora, dev, do, di, bpw):
    """One workspace for many calls: the latent kernel's slab counters are zero again after every
    call, and the results match a fresh workspace bitwise, also for a new activation."""
    r = ql.lb_rank(do, di, bpw)
    lw = ql.lb_pack(*synth.littlebit_params(do, di, r, 19, device=dev))
    ws = torch.zeros(int(ql.lib().qlinear_lb_workspace_bytes(do, di, r)), dtype=torch.uint8, device=dev)
    for seed in (21, 22):
        x = synth.activations(1, di, seed, device=dev).view(-1)
        y0 = ql.lb_gemv(x, lw)
        for _ in range(3):
            y = ql.lb_gemv(x, lw, workspace=ws)
            assert torch.equal(y, y0)
        nslab = 2 * ((r + 63) // 64)
        assert int(ws[: nslab * 128].abs().sum().item()) == 0
