"""Device code of every kernel source, compiled for gfx950 with the library's own flags, obeys
the target rules (CPU only: hipcc cross-compiles without a GPU).

- No write goes through the scalar data cache: no scalar memory stores or atomics and no
  write-back or discard of that cache (all stores are vector stores).
- No packed-fp32 VALU operation is emitted (the build turns the feature off).
- The batch-1 GEMV kernels use no scratch (their VGPRs do not spill).
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from decode_gemv_thinkbit_amd import build as qb

FORBIDDEN = re.compile(r"^\s+(s_(store|atomic|dcache_wb|dcache_discard|buffer_store|scratch_store)\w*"
                       r"|v_pk_(add|mul|fma)_f32)\b", re.M)


def device_asm(src):
    flags = [f for f in qb.FLAGS if f != "-fPIC"]
    r = subprocess.run([qb.HIPCC, *flags, "--offload-device-only", "-S", "-o", "-", os.path.join(qb.CSRC, src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(qb.HIPCC):
        pytest.skip("hipcc not available")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(qb.SOURCES))) as ex:
        return dict(zip(qb.SOURCES, ex.map(device_asm, qb.SOURCES)))


@pytest.mark.parametrize("src", qb.SOURCES)
def test_no_scalar_cache_writes_or_packed_fp32(asm, src):
    bad = FORBIDDEN.findall(asm[src])
    assert not bad, (src, sorted({b[0] for b in bad}))


def test_batch1_gemv_kernels_do_not_spill(asm):
    text = asm["ql_gemv.hip"]
    kernels = re.findall(r"^(_ZN2ql\w*gemv\w*kernel\w*):", text, re.M)
    assert kernels
    for k in kernels:
        body = text[text.index(k + ":"):]
        body = body[: body.index(".Lfunc_end")]
        assert "scratch_" not in body, k
