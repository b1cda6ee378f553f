"""The HBM read probe (needs gfx950): every byte is read exactly once.

out word 4 l + j must equal the XOR over all 1 KB blocks of dword j of bytes
16 l .. 16 l + 15, computed on the host; a second call XORs the same value in
again and returns out to zero.  Block counts that are not a multiple of the
waves' four-block unroll exercise the tail loop.
"""
import numpy as np
import pytest
import torch

from decode_gemv_thinkbit_amd import qlinear as ql

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nblk", [1, 7, 2048 + 5, 4 * 256 * 8 * 3 + 333])
def test_read_probe_reads_every_byte_once(nblk):
    assert torch.cuda.is_available()
    rng = np.random.default_rng(nblk)
    host = rng.integers(0, 2 ** 32, size=nblk * 256, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.uint8).copy()).cuda()
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    ql.read_probe(buf, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.reshape(nblk, 256), axis=0)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
    ql.read_probe(buf, out)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any()
