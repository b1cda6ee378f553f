"""ThinkBit CPU oracle (ctypes wrapper) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it and shares no code with it.

The arithmetic lives in ``thinkbit_oracle.cpp`` (plain C++17, fp64 products
and sums); this module only marshals numpy arrays.  What it computes follows
the ThinkBit summary page (onedev.kr/papers/1416), section "How it works":
w = c * s with a bf16 scale per 128 input weights and a per-layer grid of
ternary {-1,0,1}, 2-bit {-2..1} or 3-bit {-4..3}; dequantization is one
multiply.  Every function here is pinned by tests in ``tests/test_oracle_*``
against brute force, closed forms, exact rational sums or library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "thinkbit_oracle.cpp")
# ORACLE_SANITIZE=1 selects a build with AddressSanitizer and UndefinedBehaviorSanitizer (host
# code only; load it in a process that preloads the sanitizer runtime)
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle_san.so" if _SANITIZE else "liboracle.so")

GRID_T, GRID_I2, GRID_I3 = 0, 1, 2
GROUP = 128
SLAB = 64
BLOCK = 128


def build(force: bool = True) -> str:
    """Compile the oracle shared library with the host compiler."""
    if force or not os.path.exists(_LIB_PATH):
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-g"] if _SANITIZE else []
        subprocess.check_call(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-Wall", *san, "-o", tmp, _SRC,
                               "-lpthread"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.ora_cmin.argtypes = [i32]
        L.ora_cmax.argtypes = [i32]
        L.ora_f32_to_bf16.argtypes = [vp, vp, i64]
        L.ora_f32_to_bf16.restype = None
        L.ora_bf16_to_f32.argtypes = [vp, vp, i64]
        L.ora_bf16_to_f32.restype = None
        L.ora_row_bytes.argtypes = [i32, i64]
        L.ora_row_bytes.restype = i64
        L.ora_quantize.argtypes = [i64, i64, vp, vp, vp, vp]
        L.ora_requantize.argtypes = [i64, i64, vp, vp, vp, vp]
        L.ora_block_offsets.argtypes = [i64, i64, vp, vp]
        L.ora_pack.argtypes = [i64, i64, vp, vp, vp]
        L.ora_unpack.argtypes = [i64, i64, vp, vp, vp]
        L.ora_packed_scales_len.argtypes = [i64, i64]
        L.ora_packed_scales_len.restype = i64
        L.ora_pack_scales.argtypes = [i64, i64, vp, vp]
        L.ora_unpack_scales.argtypes = [i64, i64, vp, vp]
        L.ora_dequant.argtypes = [i64, i64, vp, vp, vp, vp]
        L.ora_dequant.restype = None
        L.ora_gemv.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32]
        L.ora_gemv.restype = None
        L.ora_gemv_w16.argtypes = [i64, i64, i64, vp, vp, vp, vp, i32]
        L.ora_gemv_w16.restype = None
        L.ora_c4_bytes.argtypes = [i64, i64]
        L.ora_c4_bytes.restype = i64
        L.ora_c4_pack.argtypes = [i64, i64, vp, vp]
        L.ora_c4_unpack.argtypes = [i64, i64, vp, vp]
        L.ora_lb_bpw.argtypes = [i64, i64, i64]
        L.ora_lb_bpw.restype = ctypes.c_double
        L.ora_lb_rank.argtypes = [i64, i64, ctypes.c_double]
        L.ora_lb_rank.restype = i64
        L.ora_lb_u_bytes.argtypes = [i64, i64]
        L.ora_lb_u_bytes.restype = i64
        L.ora_lb_v_bytes.argtypes = [i64, i64]
        L.ora_lb_v_bytes.restype = i64
        L.ora_lb_pack.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.ora_lb_unpack.argtypes = [i64, i64, i64, vp, vp, vp, vp]
        L.ora_lb_gemv.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.ora_rtn_noise.argtypes = [i64, i64, vp, vp]
        L.ora_block_sensitivity.argtypes = [i64, vp, i64, vp, vp]
        L.ora_allocate.argtypes = [i64, vp, vp, vp, vp, vp, ctypes.c_double, vp, vp]
        L.ora_gemv_packed.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def cmin(grid: int) -> int:
    return lib().ora_cmin(grid)


def cmax(grid: int) -> int:
    return lib().ora_cmax(grid)


def f32_to_bf16(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().ora_f32_to_bf16(_p(a), _p(out), a.size)
    return out


def bf16_to_f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float32)
    lib().ora_bf16_to_f32(_p(a), _p(out), a.size)
    return out


def row_bytes(grid: int, K: int) -> int:
    return int(lib().ora_row_bytes(grid, K))


def n_blocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def row_grids(N: int, blk_grid) -> np.ndarray:
    """Grid of every row from the per-128-row block table."""
    blk_grid = np.asarray(blk_grid, dtype=np.int8)
    return np.ascontiguousarray(np.repeat(blk_grid, BLOCK)[:N])


def _blk(N: int, grid_or_table) -> np.ndarray:
    if np.isscalar(grid_or_table):
        return np.full(n_blocks(N), int(grid_or_table), dtype=np.int8)
    t = np.ascontiguousarray(grid_or_table, dtype=np.int8)
    assert t.shape == (n_blocks(N),)
    return t


def quantize(W: np.ndarray, grid) -> tuple[np.ndarray, np.ndarray]:
    """Round-to-nearest codes int8 [N][K] and bf16 scale bits [N][K/128]."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    rg = row_grids(N, _blk(N, grid))
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, K // GROUP), dtype=np.uint16)
    rc = lib().ora_quantize(N, K, _p(rg), _p(W), _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("oracle quantize rejected its input")
    return codes, scales


def requantize(W: np.ndarray, scales: np.ndarray, grid) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.float32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = W.shape
    rg = row_grids(N, _blk(N, grid))
    codes = np.empty((N, K), dtype=np.int8)
    if lib().ora_requantize(N, K, _p(rg), _p(W), _p(scales), _p(codes)) != 0:
        raise ValueError("oracle requantize rejected its input")
    return codes


def block_offsets(N: int, K: int, grid) -> np.ndarray:
    t = _blk(N, grid)
    off = np.empty(len(t) + 1, dtype=np.int64)
    if lib().ora_block_offsets(N, K, _p(t), _p(off)) != 0:
        raise ValueError("bad shape or grid")
    return off


def pack(codes: np.ndarray, grid) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    t = _blk(N, grid)
    out = np.empty(int(block_offsets(N, K, t)[-1]), dtype=np.uint8)
    if lib().ora_pack(N, K, _p(t), _p(codes), _p(out)) != 0:
        raise ValueError("bad shape or grid")
    return out


def unpack(packed: np.ndarray, N: int, K: int, grid) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    t = _blk(N, grid)
    codes = np.empty((N, K), dtype=np.int8)
    rc = lib().ora_unpack(N, K, _p(t), _p(packed), _p(codes))
    if rc == -2:
        raise ValueError("invalid ternary byte (> 242)")
    if rc != 0:
        raise ValueError("bad shape or grid")
    return codes


def c4_pack(codes: np.ndarray) -> np.ndarray:
    """Codes [N][K] (each in -8..7) -> the 4-bit container (two's complement nibbles,
    lower input in the low nibble, 64-row slab interleave as the packed layout)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    out = np.empty(int(lib().ora_c4_bytes(N, K)), dtype=np.uint8)
    rc = lib().ora_c4_pack(N, K, _p(codes), _p(out))
    if rc == -3:
        raise ValueError("code outside -8..7")
    if rc != 0:
        raise ValueError("bad shape")
    return out


def c4_unpack(c4: np.ndarray, N: int, K: int) -> np.ndarray:
    c4 = np.ascontiguousarray(c4, dtype=np.uint8)
    codes = np.empty((N, K), dtype=np.int8)
    if lib().ora_c4_unpack(N, K, _p(c4), _p(codes)) != 0:
        raise ValueError("bad shape")
    return codes


def pack_scales(scales: np.ndarray, K: int) -> np.ndarray:
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N = scales.shape[0]
    out = np.empty(int(lib().ora_packed_scales_len(N, K)), dtype=np.uint16)
    if lib().ora_pack_scales(N, K, _p(scales), _p(out)) != 0:
        raise ValueError("bad shape")
    return out


def unpack_scales(ps: np.ndarray, N: int, K: int) -> np.ndarray:
    ps = np.ascontiguousarray(ps, dtype=np.uint16)
    out = np.empty((N, K // GROUP), dtype=np.uint16)
    if lib().ora_unpack_scales(N, K, _p(ps), _p(out)) != 0:
        raise ValueError("bad shape")
    return out


def dequant(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """w32 = c*s (fp32, exact) and w16 = bf16_rne(w32) bits."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    N, K = codes.shape
    w32 = np.empty((N, K), dtype=np.float32)
    w16 = np.empty((N, K), dtype=np.uint16)
    lib().ora_dequant(N, K, _p(codes), _p(scales), _p(w32), _p(w16))
    return w32, w16


def gemv(codes: np.ndarray, scales: np.ndarray, x_bf16: np.ndarray, threads: int = 0) -> np.ndarray:
    """y64 [M][N] = sum_k (c*s)[n,k] * x[m,k] in fp64 (ascending k)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x = np.ascontiguousarray(np.atleast_2d(x_bf16), dtype=np.uint16)
    N, K = codes.shape
    M = x.shape[0]
    assert x.shape[1] == K
    y = np.empty((M, N), dtype=np.float64)
    lib().ora_gemv(M, N, K, _p(codes), _p(scales), _p(x), _p(y), threads or (os.cpu_count() or 1))
    return y


def gemv_w16(codes: np.ndarray, scales: np.ndarray, x_bf16: np.ndarray, threads: int = 0) -> np.ndarray:
    """y [M][N] = sum_k bf16_rne(c*s)[n,k] * x[m,k] in fp64 (ascending k): the product with
    weights dequantized to bf16, equal to gemv wherever c*s is a bf16 value."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x = np.ascontiguousarray(np.atleast_2d(x_bf16), dtype=np.uint16)
    N, K = codes.shape
    M = x.shape[0]
    assert x.shape[1] == K
    y = np.empty((M, N), dtype=np.float64)
    lib().ora_gemv_w16(M, N, K, _p(codes), _p(scales), _p(x), _p(y), threads or (os.cpu_count() or 1))
    return y


def gemv_packed(packed: np.ndarray, pscales: np.ndarray, x_bf16: np.ndarray, N: int, K: int, grid,
                threads: int = 0) -> np.ndarray:
    """The same product read from the packed buffers with the oracle's own decoder."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    pscales = np.ascontiguousarray(pscales, dtype=np.uint16)
    x = np.ascontiguousarray(np.atleast_2d(x_bf16), dtype=np.uint16)
    M = x.shape[0]
    t = _blk(N, grid)
    y = np.empty((M, N), dtype=np.float64)
    rc = lib().ora_gemv_packed(M, N, K, _p(t), _p(packed), _p(pscales), _p(x), _p(y),
                               threads or (os.cpu_count() or 1))
    if rc != 0:
        raise ValueError("oracle gemv_packed failed (%d)" % rc)
    return y


def rel_err(y_gpu: np.ndarray, y64: np.ndarray) -> tuple[float, float]:
    """(max over token rows of max_n|dy| / ||y64 row||_2, normwise ||dy||/||y64||)."""
    y_gpu = np.atleast_2d(np.asarray(y_gpu, dtype=np.float64))
    y64 = np.atleast_2d(y64)
    d = y_gpu - y64
    rown = np.linalg.norm(y64, axis=1)
    rown = np.where(rown == 0, 1.0, rown)
    per_row = np.max(np.abs(d), axis=1) / rown
    tot = np.linalg.norm(y64)
    return float(per_row.max()), float(np.linalg.norm(d) / (tot if tot else 1.0))


# ---------------------------------------------------------------- grid allocation
# Bits per weight of each grid for the budget: code bits plus one bf16 scale per
# 128 weights; ternary carries log2(3) bits of information per code.
GRID_BITS = np.array([np.log2(3.0) + 16 / 128, 2 + 16 / 128, 3 + 16 / 128])


def rtn_noise(W: np.ndarray) -> np.ndarray:
    """[ceil(N/128)][3]: sum over each 128-row block of (w - c*s)^2 for the T, I2, I3
    round-to-nearest quantizations (fp64)."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    out = np.empty((n_blocks(N), 3), dtype=np.float64)
    if lib().ora_rtn_noise(N, K, _p(W), _p(out)) != 0:
        raise ValueError("bad shape or non-finite weight")
    return out


def block_sensitivity(x_bf16: np.ndarray, grad: np.ndarray) -> np.ndarray:
    """S per 128-row block: ||x||^2 * sum of the block's squared output gradients (fp64)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1)
    g = np.ascontiguousarray(grad, dtype=np.float32).reshape(-1)
    out = np.empty(n_blocks(len(g)), dtype=np.float64)
    if lib().ora_block_sensitivity(len(x), _p(x), len(g), _p(g), _p(out)) != 0:
        raise ValueError("bad shape")
    return out


def allocate(n, S, E, allowed, budget: float, bits=None) -> tuple[np.ndarray, float]:
    """Lagrangian multiple-choice knapsack by the convex-hull greedy: grid per unit and the
    slope of the first group of hull edges left out (0 when every edge fits)."""
    n = np.ascontiguousarray(n, dtype=np.int64)
    S = np.ascontiguousarray(S, dtype=np.float64)
    E = np.ascontiguousarray(E, dtype=np.float64).reshape(len(n), 3)
    allowed = np.ascontiguousarray(allowed, dtype=np.uint32)
    bits = np.ascontiguousarray(GRID_BITS if bits is None else bits, dtype=np.float64)
    out = np.empty(len(n), dtype=np.int8)
    lam = ctypes.c_double(0.0)
    rc = lib().ora_allocate(len(n), _p(n), _p(S), _p(E), _p(allowed), _p(bits), float(budget), _p(out),
                            ctypes.byref(lam))
    if rc == -2:
        raise ValueError("budget below the cheapest allowed grids")
    if rc != 0:
        raise ValueError("bad allocation input")
    return out, lam.value


# ---------------------------------------------------------------- LittleBit
def lb_bpw(d_out: int, d_in: int, r: int) -> float:
    return float(lib().ora_lb_bpw(d_out, d_in, r))


def lb_rank(d_out: int, d_in: int, bpw: float) -> int:
    return int(lib().ora_lb_rank(d_out, d_in, float(bpw)))


def lb_pack(u_signs: np.ndarray, v_signs: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """u_signs int8 [2][d_out][r], v_signs int8 [2][d_in][r] (+-1) -> (u_bits, v_bits)."""
    u = np.ascontiguousarray(u_signs, dtype=np.int8)
    v = np.ascontiguousarray(v_signs, dtype=np.int8)
    _, d_out, r = u.shape
    d_in = v.shape[1]
    ub = np.empty(int(lib().ora_lb_u_bytes(d_out, r)), np.uint8)
    vb = np.empty(int(lib().ora_lb_v_bytes(d_in, r)), np.uint8)
    rc = lib().ora_lb_pack(d_out, d_in, r, _p(u), _p(v), _p(ub), _p(vb))
    if rc == -3:
        raise ValueError("sign other than +-1")
    if rc != 0:
        raise ValueError("bad shape")
    return ub, vb


def lb_unpack(u_bits: np.ndarray, v_bits: np.ndarray, d_out: int, d_in: int, r: int):
    u = np.empty((2, d_out, r), np.int8)
    v = np.empty((2, d_in, r), np.int8)
    if lib().ora_lb_unpack(d_out, d_in, r, _p(np.ascontiguousarray(u_bits, np.uint8)),
                           _p(np.ascontiguousarray(v_bits, np.uint8)), _p(u), _p(v)) != 0:
        raise ValueError("bad shape")
    return u, v


def lb_gemv(u_signs, v_signs, g, l, h, x) -> np.ndarray:
    """fp64 y [d_out] of the two-path LittleBit linear at batch 1 (bf16 bits for g, l, h, x)."""
    u = np.ascontiguousarray(u_signs, dtype=np.int8)
    v = np.ascontiguousarray(v_signs, dtype=np.int8)
    _, d_out, r = u.shape
    d_in = v.shape[1]
    y = np.empty(d_out, np.float64)
    arrs = [np.ascontiguousarray(a, dtype=np.uint16) for a in (g, l, h, x)]
    if lib().ora_lb_gemv(d_out, d_in, r, _p(u), _p(v), *[_p(a) for a in arrs], _p(y)) != 0:
        raise ValueError("bad shape")
    return y
