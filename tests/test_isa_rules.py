"""Device code of every kernel source, compiled for gfx950 with the library's own flags, obeys
the target rules (CPU only: hipcc cross-compiles without a GPU).

- No write goes through the scalar data cache: no scalar memory stores or atomics and no
  write-back or discard of that cache (all stores are vector stores).
- No packed-fp32 VALU operation is emitted (the build turns the feature off).
- The GEMV kernels use no scratch (their VGPRs do not spill); every other kernel's
  private segment stays within a stated bound (at present zero for every kernel).
- The split-K protocol (a part's partial sums stored at agent scope, a wait for those
  stores, then an agent-scope counter increment; the last part loads the partials at agent
  scope) is emitted with those properties: agent-scope stores and loads carry sc1 (they go
  to and come from L2, which every CU of the device shares), the counter atomics return
  their old value (sc0), and no counter atomic follows an agent-scope store without an
  intervening vmcnt(0) wait.
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


def test_gemv_kernels_do_not_spill(asm):
    text = asm["ql_gemv.hip"]
    kernels = re.findall(r"^(_ZN2ql\w*gemv\w*kernel\w*):", text, re.M)
    assert len(kernels) >= 8  # single-matrix and grouped, four token-group counts each
    for k in kernels:
        body = text[text.index(k + ":"):]
        body = body[: body.index(".Lfunc_end")]
        assert "scratch_" not in body, k


def kernel_bodies(text):
    """name -> assembly of each kernel in one compiled source."""
    out = {}
    for k in re.findall(r"^(_ZN2ql\w*kernel\w*):", text, re.M):
        body = text[text.index(k + ":"):]
        out[k] = body[: body.index(".Lfunc_end")]
    return out


def kernel_metadata(text):
    """name -> private segment bytes, from the code object's metadata."""
    meta = text[text.index(".amdgpu_metadata"): text.index(".end_amdgpu_metadata")]
    out = {}
    for entry in meta.split("\n  - ")[1:]:
        name = re.search(r"^\s+\.name:\s+(\S+)", entry, re.M)
        priv = re.search(r"^\s+\.private_segment_fixed_size:\s+(\d+)", entry, re.M)
        if name and priv:
            out[name.group(1)] = int(priv.group(1))
    return out


# Largest private segment (bytes per lane) a kernel may use; kernels not listed use none.
SCRATCH_BOUND = {}


@pytest.mark.parametrize("src", qb.SOURCES)
def test_private_segment_bounds(asm, src):
    meta = kernel_metadata(asm[src])
    assert meta or src == "ql_api.hip", src
    for name, priv in meta.items():
        bound = next((b for key, b in SCRATCH_BOUND.items() if key in name), 0)
        assert priv <= bound, (src, name, priv, bound)


# Kernels that run the split-K protocol (or its LittleBit form) and where they are compiled.
SPLIT_KERNELS = [("ql_gemv.hip", "gemv_grouped_kernel"), ("ql_c4.hip", "c4_gemv_grouped_kernel"),
                 ("ql_littlebit.hip", "lb_latent_kernel")]
STORE_SC1 = re.compile(r"^\s+(global|flat)_store_dword\w*\s[^;\n]*\bsc1\b", re.M)
LOAD_SC1 = re.compile(r"^\s+(global|flat)_load_dword\w*\s[^;\n]*\bsc1\b", re.M)


@pytest.mark.parametrize("src,kernel", SPLIT_KERNELS)
def test_split_protocol_scope_bits(asm, src, kernel):
    bodies = {k: b for k, b in kernel_bodies(asm[src]).items() if kernel in k}
    assert bodies, (src, kernel)
    for name, body in bodies.items():
        assert STORE_SC1.search(body), (name, "no agent-scope store")
        assert LOAD_SC1.search(body), (name, "no agent-scope load")
        pending = None
        for line in body.split("\n"):
            code = line.split(";")[0]
            m = re.match(r"\s+((global|flat)_atomic\w*)(.*)", code)
            if STORE_SC1.match(code):
                pending = code.strip()
            elif re.match(r"\s+s_waitcnt\b.*\bvmcnt\(0\)", code):
                pending = None
            elif m:
                assert re.search(r"\bsc0\b", m.group(3)), (name, "atomic without return", code.strip())
                assert pending is None, (name, "counter atomic after an unwaited store", pending, code.strip())
