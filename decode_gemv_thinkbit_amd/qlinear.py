"""Thin Python binding of libqlinear.so (argument marshalling only).

Every step of the path runs in the HIP kernels behind the C ABI declared in
``include/qlinear.h``; this module only checks tensor dtypes/devices, passes
raw device pointers and the current torch stream, and maps status codes to
exceptions.  There is no fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

GRID_T, GRID_I2, GRID_I3, GRID_MIXED = 0, 1, 2, 3
GRID_C4 = 4  # 4-bit container baseline (not a ThinkBit grid)
GROUP, SLAB, BLOCK = 128, 64, 128
QL_SCHED_WORDS = 4128  # uint32 words of grouped-launch scheduler state
QL_MAX_KPARTS = 16  # split-K parts per slab at most
QL_NOALLOC_STATE_WORDS = 4194304  # uint32 words of the library's static grouped-launch state

_HERE = os.path.dirname(os.path.abspath(__file__))
# QLINEAR_SANITIZE=1 loads the build whose host code carries AddressSanitizer and
# UndefinedBehaviorSanitizer (decode_gemv_thinkbit_amd/build.py); the process must preload
# clang's ASan runtime
LIB_PATH = os.path.join(_HERE, "_build_san" if os.environ.get("QLINEAR_SANITIZE") == "1" else "_build",
                        "libqlinear.so")

_lib = None


class QLinearError(RuntimeError):
    pass


class ql_gemv_desc(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("pscales", ctypes.c_void_p), ("blk_grid", ctypes.c_void_p),
                ("blk_off", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("slab_begin", ctypes.c_int32), ("kparts", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ws_begin", ctypes.c_int64)]


class ql_alloc_unit(ctypes.Structure):
    _fields_ = [("weights", ctypes.c_int64), ("sensitivity", ctypes.c_double), ("noise", ctypes.c_double * 3),
                ("allowed", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class ql_littlebit(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int32), ("d_in", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("u_bits", ctypes.c_void_p), ("v_bits", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("l", ctypes.c_void_p), ("h", ctypes.c_void_p)]


def lib():
    """Load libqlinear.so; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise QLinearError(f"HIP library not built: {LIB_PATH} (run decode_gemv_thinkbit_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.qlinear_version.restype = i32
        L.qlinear_last_error.restype = ctypes.c_char_p
        L.qlinear_row_bytes.argtypes = [i32, i64]
        L.qlinear_row_bytes.restype = i64
        L.qlinear_block_offsets.argtypes = [i64, i64, vp, vp]
        L.qlinear_packed_bytes.argtypes = [i64, i64, i32]
        L.qlinear_packed_bytes.restype = i64
        L.qlinear_packed_scales_len.argtypes = [i64, i64]
        L.qlinear_packed_scales_len.restype = i64
        L.qlinear_quantize.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        L.qlinear_pack.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
        L.qlinear_pack_scales.argtypes = [i64, i64, vp, vp, vp]
        L.qlinear_unpack.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        L.qlinear_unpack_scales.argtypes = [i64, i64, vp, vp, vp]
        L.qlinear_dequant.argtypes = [i64, i64, i32, vp, vp, vp, vp, i32, vp, vp]
        L.qlinear_gemv.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp]
        L.qlinear_grouped_prepare.argtypes = [vp, ctypes.c_int32]
        L.qlinear_grouped_prepare.restype = i64
        L.qlinear_grouped_prepare_split.argtypes = [vp, ctypes.c_int32, i64, ctypes.POINTER(i64)]
        L.qlinear_grouped_prepare_split.restype = i64
        L.qlinear_read_probe.argtypes = [vp, i64, vp, vp]
        L.qlinear_read_probe.restype = ctypes.c_int
        L.qlinear_grouped_wave_slots.argtypes = [ctypes.c_int32]
        L.qlinear_grouped_wave_slots.restype = i64
        L.qlinear_gemv_grouped.argtypes = [vp, ctypes.c_int32, i64, ctypes.c_int32, vp, vp]
        L.qlinear_gemv_grouped_noalloc.argtypes = [vp, ctypes.c_int32, i64, ctypes.c_int32, i64, vp]
        L.qlinear_gemm_workspace_bytes.argtypes = [i64, i64, i64]
        L.qlinear_gemm_workspace_bytes.restype = sz
        L.qlinear_gemm.argtypes = [i64, i64, i64, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.qlinear_gemm_grouped_prepare.argtypes = [vp, ctypes.c_int32, i64, ctypes.POINTER(i64)]
        L.qlinear_gemm_grouped_prepare.restype = i64
        L.qlinear_gemm_grouped.argtypes = [vp, ctypes.c_int32, i64, i64, vp, sz, vp]
        L.qlinear_rtn_noise.argtypes = [i64, i64, vp, vp, vp]
        L.qlinear_allocate.argtypes = [vp, i64, ctypes.c_double, vp, vp, vp]
        L.qlinear_block_sensitivity.argtypes = [i64, i64, vp, vp, vp, vp]
        L.qlinear_validate_codes.argtypes = [i64, i64, i32, vp, vp, vp, vp]
        L.qlinear_validate_packed.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        L.qlinear_lb_bpw.argtypes = [i64, i64, i64]
        L.qlinear_lb_bpw.restype = ctypes.c_double
        L.qlinear_lb_rank.argtypes = [i64, i64, ctypes.c_double]
        L.qlinear_lb_rank.restype = i64
        L.qlinear_lb_u_bytes.argtypes = [i64, i64]
        L.qlinear_lb_u_bytes.restype = i64
        L.qlinear_lb_v_bytes.argtypes = [i64, i64]
        L.qlinear_lb_v_bytes.restype = i64
        L.qlinear_lb_pack.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        L.qlinear_lb_workspace_bytes.argtypes = [i64, i64, i64]
        L.qlinear_lb_workspace_bytes.restype = sz
        L.qlinear_lb_gemv.argtypes = [vp, vp, vp, vp, sz, vp]
        L.qlinear_c4_bytes.argtypes = [i64, i64]
        L.qlinear_c4_bytes.restype = i64
        L.qlinear_c4_pack.argtypes = [i64, i64, vp, vp, vp]
        L.qlinear_c4_unpack.argtypes = [i64, i64, vp, vp, vp]
        L.qlinear_c4_to_packed.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        L.qlinear_c4_gemv.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        L.qlinear_c4_gemv_grouped.argtypes = [vp, ctypes.c_int32, i64, ctypes.c_int32, vp, vp]
        for name in ("qlinear_block_offsets", "qlinear_quantize", "qlinear_pack", "qlinear_pack_scales",
                     "qlinear_unpack", "qlinear_unpack_scales", "qlinear_dequant", "qlinear_gemv",
                     "qlinear_gemv_grouped", "qlinear_gemv_grouped_noalloc", "qlinear_gemm", "qlinear_gemm_grouped", "qlinear_c4_pack", "qlinear_c4_unpack",
                     "qlinear_c4_to_packed", "qlinear_c4_gemv", "qlinear_c4_gemv_grouped", "qlinear_rtn_noise",
                     "qlinear_allocate", "qlinear_block_sensitivity", "qlinear_validate_codes", "qlinear_validate_packed", "qlinear_lb_pack", "qlinear_lb_gemv"):
            getattr(L, name).restype = i32
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != 0:
        raise QLinearError(f"{what}: status {status}: {lib().qlinear_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ---------------------------------------------------------------- sizes
def row_bytes(grid: int, K: int) -> int:
    return int(lib().qlinear_row_bytes(grid, K))


def n_blocks(N: int) -> int:
    return (N + BLOCK - 1) // BLOCK


def block_offsets(N: int, K: int, blk_grid) -> np.ndarray:
    t = np.ascontiguousarray(blk_grid, dtype=np.int8)
    if t.shape != (n_blocks(N),):
        raise ValueError("blk_grid needs one entry per 128-row block")
    off = np.empty(len(t) + 1, dtype=np.int64)
    _check(lib().qlinear_block_offsets(N, K, t.ctypes.data_as(ctypes.c_void_p), off.ctypes.data_as(ctypes.c_void_p)),
           "block_offsets")
    return off


def packed_scales_len(N: int, K: int) -> int:
    return int(lib().qlinear_packed_scales_len(N, K))


@dataclass
class PackedWeight:
    """A ThinkBit weight in the library's packed layout (device tensors)."""
    packed: torch.Tensor      # uint8, packed codes
    pscales: torch.Tensor     # bfloat16, packed scale array
    N: int
    K: int
    grid: int                 # GRID_T/I2/I3 or GRID_MIXED
    blk_grid: Optional[torch.Tensor] = None  # int8 [ceil(N/128)] on device (mixed only)
    blk_off: Optional[torch.Tensor] = None   # int64 [ceil(N/128)+1] on device (mixed only)

    @property
    def nbytes(self) -> int:
        """Stored bytes of codes and scales (padding included)."""
        return self.packed.numel() + 2 * self.pscales.numel()


def _grid_tables(N: int, K: int, grid, device):
    """(grid id, blk_grid dev tensor or None, blk_off dev tensor or None, packed size)."""
    if isinstance(grid, (int, np.integer)):
        g = int(grid)
        size = int(lib().qlinear_packed_bytes(N, K, g))
        if size <= 0:
            raise ValueError(f"invalid grid {g} or shape {N}x{K}")
        return g, None, None, size
    table = np.ascontiguousarray(np.asarray(grid), dtype=np.int8)
    off = block_offsets(N, K, table)
    bg = torch.from_numpy(table).to(device)
    bo = torch.from_numpy(off).to(device)
    return GRID_MIXED, bg, bo, int(off[-1])


# ---------------------------------------------------------------- quantize / pack
def quantize(W: torch.Tensor, grid) -> tuple[torch.Tensor, torch.Tensor]:
    """Round-to-nearest codes (int8 [N,K]) and bf16 scales [N, K/128] on the device."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    g, bg, _, _ = _grid_tables(N, K, grid, W.device)
    codes = torch.empty((N, K), dtype=torch.int8, device=W.device)
    scales = torch.empty((N, K // GROUP), dtype=torch.bfloat16, device=W.device)
    _check(lib().qlinear_quantize(N, K, g, _ptr(bg), _ptr(W), _ptr(codes), _ptr(scales), _stream()), "quantize")
    return codes, scales


def pack(codes: torch.Tensor, scales: torch.Tensor, grid, packed: Optional[torch.Tensor] = None,
         pscales: Optional[torch.Tensor] = None) -> PackedWeight:
    """Codes int8 [N, K] and bf16 scales [N, K/128] -> the packed layout (one qlinear_pack call).
    packed / pscales: optional preallocated outputs (uint8 of the packed size, bf16 of
    packed_scales_len elements), e.g. views into one arena holding a whole model."""
    _dev(codes, torch.int8, "codes")
    _dev(scales, torch.bfloat16, "scales")
    N, K = codes.shape
    if tuple(scales.shape) != (N, K // GROUP):
        raise ValueError("scales must be [N, K/128]")
    g, bg, bo, size = _grid_tables(N, K, grid, codes.device)
    if packed is None:
        packed = torch.empty(size, dtype=torch.uint8, device=codes.device)
    elif packed.dtype != torch.uint8 or packed.numel() != size or not packed.is_contiguous():
        raise ValueError(f"packed must be a contiguous uint8 tensor of {size} bytes")
    plen = packed_scales_len(N, K)
    if pscales is None:
        pscales = torch.empty(plen, dtype=torch.bfloat16, device=codes.device)
    elif pscales.dtype != torch.bfloat16 or pscales.numel() != plen or not pscales.is_contiguous():
        raise ValueError(f"pscales must be a contiguous bf16 tensor of {plen} elements")
    _check(lib().qlinear_pack(N, K, g, _ptr(bg), _ptr(bo), _ptr(codes), _ptr(scales), _ptr(packed),
                              _ptr(pscales), _stream()), "pack")
    return PackedWeight(packed, pscales, N, K, g, bg, bo)


def packed_sizes(N: int, K: int, grid) -> tuple[int, int]:
    """(packed code bytes, packed scale elements) of an N x K weight on `grid` (int or per-block table)."""
    if isinstance(grid, (int, np.integer)):
        size = int(lib().qlinear_packed_bytes(N, K, int(grid)))
    else:
        size = int(block_offsets(N, K, np.asarray(grid))[-1])
    return size, packed_scales_len(N, K)


def quantize_pack(W: torch.Tensor, grid, packed: Optional[torch.Tensor] = None,
                  pscales: Optional[torch.Tensor] = None) -> PackedWeight:
    codes, scales = quantize(W, grid)
    return pack(codes, scales, grid, packed, pscales)


def validate_codes(codes: torch.Tensor, grid) -> np.ndarray:
    """Counts [codes outside their grid, -, bad block grids, -] of int8 codes [N, K] (device).
    grid: a grid id, or a per-block table (uploaded as is, unchecked on the host)."""
    _dev(codes, torch.int8, "codes")
    N, K = codes.shape
    bg = None
    if isinstance(grid, (int, np.integer)):
        g = int(grid)
    else:
        g = GRID_MIXED
        bg = torch.from_numpy(np.ascontiguousarray(grid, dtype=np.int8)).to(codes.device)
    out = torch.zeros(4, dtype=torch.int32, device=codes.device)
    _check(lib().qlinear_validate_codes(N, K, g, _ptr(bg), _ptr(codes), _ptr(out), _stream()), "validate_codes")
    return out.cpu().numpy()


def validate_packed(pw: PackedWeight) -> np.ndarray:
    """Counts [ternary bytes above 242, padding not coding 0, bad block grids, -] of a packed weight."""
    out = torch.zeros(4, dtype=torch.int32, device=pw.packed.device)
    _check(lib().qlinear_validate_packed(pw.N, pw.K, pw.grid, _ptr(pw.blk_grid), _ptr(pw.blk_off), _ptr(pw.packed),
                                         _ptr(out), _stream()), "validate_packed")
    return out.cpu().numpy()


def unpack(pw: PackedWeight) -> torch.Tensor:
    codes = torch.empty((pw.N, pw.K), dtype=torch.int8, device=pw.packed.device)
    _check(lib().qlinear_unpack(pw.N, pw.K, pw.grid, _ptr(pw.blk_grid), _ptr(pw.blk_off), _ptr(pw.packed),
                                _ptr(codes), _stream()), "unpack")
    return codes


def unpack_scales(pw: PackedWeight) -> torch.Tensor:
    s = torch.empty((pw.N, pw.K // GROUP), dtype=torch.bfloat16, device=pw.packed.device)
    _check(lib().qlinear_unpack_scales(pw.N, pw.K, _ptr(pw.pscales), _ptr(s), _stream()), "unpack_scales")
    return s


def dequant(pw: PackedWeight, out_bf16: bool = False) -> torch.Tensor:
    out = torch.empty((pw.N, pw.K), dtype=torch.bfloat16 if out_bf16 else torch.float32, device=pw.packed.device)
    _check(lib().qlinear_dequant(pw.N, pw.K, pw.grid, _ptr(pw.blk_grid), _ptr(pw.blk_off), _ptr(pw.packed),
                                 _ptr(pw.pscales), 1 if out_bf16 else 0, _ptr(out), _stream()), "dequant")
    return out


# ---------------------------------------------------------------- grid allocation (offline)
ALL_GRIDS, AT_LEAST_2BIT = 0b111, 0b110  # allowed-grid masks


def rtn_noise(W: torch.Tensor) -> torch.Tensor:
    """float64 [ceil(N/128), 3] on the device: per 128-row block, sum of (w - c*s)^2 of the
    round-to-nearest quantization onto T, I2, I3."""
    _dev(W, torch.float32, "W")
    N, K = W.shape
    out = torch.empty((n_blocks(N), 3), dtype=torch.float64, device=W.device)
    _check(lib().qlinear_rtn_noise(N, K, _ptr(W), _ptr(out), _stream()), "rtn_noise")
    return out


def block_sensitivity(x: torch.Tensor, grad: torch.Tensor) -> torch.Tensor:
    """float64 [ceil(N/128)] on the device: ||x||^2 * (sum of grad^2 over each 128-row block)."""
    _dev(x, torch.bfloat16, "x")
    _dev(grad, torch.float32, "grad")
    K, N = x.numel(), grad.numel()
    out = torch.empty(n_blocks(N), dtype=torch.float64, device=x.device)
    _check(lib().qlinear_block_sensitivity(N, K, _ptr(x), _ptr(grad), _ptr(out), _stream()), "block_sensitivity")
    return out


def allocate(weights, sensitivity, noise, allowed, budget_bits: float, grid_bits=None):
    """Lagrangian multiple-choice knapsack over units (host): (grid per unit int8, multiplier)."""
    weights = np.asarray(weights, dtype=np.int64)
    count = len(weights)
    sensitivity = np.asarray(sensitivity, dtype=np.float64).reshape(count)
    noise = np.asarray(noise, dtype=np.float64).reshape(count, 3)
    allowed = np.broadcast_to(np.asarray(allowed, dtype=np.uint32), (count,))
    units = (ql_alloc_unit * count)()
    for i in range(count):
        units[i].weights = int(weights[i])
        units[i].sensitivity = float(sensitivity[i])
        for g in range(3):
            units[i].noise[g] = float(noise[i, g])
        units[i].allowed = int(allowed[i])
    out = np.empty(count, dtype=np.int8)
    lam = ctypes.c_double(0.0)
    bits = None if grid_bits is None else np.ascontiguousarray(grid_bits, dtype=np.float64)
    _check(lib().qlinear_allocate(ctypes.cast(units, ctypes.c_void_p), count, float(budget_bits),
                                  None if bits is None else bits.ctypes.data_as(ctypes.c_void_p),
                                  out.ctypes.data_as(ctypes.c_void_p), ctypes.byref(lam)), "allocate")
    return out, lam.value


# ---------------------------------------------------------------- LittleBit (binary factorized)
def lb_bpw(d_out: int, d_in: int, rank: int) -> float:
    return float(lib().qlinear_lb_bpw(d_out, d_in, rank))


def lb_rank(d_out: int, d_in: int, bpw: float) -> int:
    return int(lib().qlinear_lb_rank(d_out, d_in, float(bpw)))


@dataclass
class LittleBitWeight:
    """A two-path LittleBit linear: packed signs and bf16 scales on the device."""
    u_bits: torch.Tensor   # uint8
    v_bits: torch.Tensor   # uint8
    g: torch.Tensor        # bf16 [2, d_in]
    l: torch.Tensor        # bf16 [2, rank]
    h: torch.Tensor        # bf16 [2, d_out]
    d_out: int
    d_in: int
    rank: int

    @property
    def nbytes(self) -> int:
        """Stored bytes: sign buffers (padding included) and the three scale vectors."""
        return self.u_bits.numel() + self.v_bits.numel() + 2 * (self.g.numel() + self.l.numel() + self.h.numel())

    def desc(self) -> ql_littlebit:
        return ql_littlebit(self.d_out, self.d_in, self.rank, 0, self.u_bits.data_ptr(), self.v_bits.data_ptr(),
                            self.g.data_ptr(), self.l.data_ptr(), self.h.data_ptr())


def lb_pack(u_signs: torch.Tensor, v_signs: torch.Tensor, g: torch.Tensor, l: torch.Tensor,
            h: torch.Tensor) -> LittleBitWeight:
    """u_signs int8 [2, d_out, r], v_signs int8 [2, d_in, r] (+-1); g, l, h bf16 [2, *]."""
    _dev(u_signs, torch.int8, "u_signs")
    _dev(v_signs, torch.int8, "v_signs")
    for t, name in ((g, "g"), (l, "l"), (h, "h")):
        _dev(t, torch.bfloat16, name)
    _, d_out, r = u_signs.shape
    d_in = v_signs.shape[1]
    if tuple(v_signs.shape) != (2, d_in, r) or tuple(g.shape) != (2, d_in) or tuple(l.shape) != (2, r) or \
            tuple(h.shape) != (2, d_out):
        raise ValueError("inconsistent LittleBit shapes")
    ub = int(lib().qlinear_lb_u_bytes(d_out, r))
    vb = int(lib().qlinear_lb_v_bytes(d_in, r))
    if ub <= 0 or vb <= 0:
        raise ValueError(f"invalid LittleBit shape {d_out}x{d_in}, rank {r}")
    u_bits = torch.empty(ub, dtype=torch.uint8, device=u_signs.device)
    v_bits = torch.empty(vb, dtype=torch.uint8, device=u_signs.device)
    _check(lib().qlinear_lb_pack(d_out, d_in, r, _ptr(u_signs), _ptr(v_signs), _ptr(u_bits), _ptr(v_bits),
                                 _stream()), "lb_pack")
    return LittleBitWeight(u_bits, v_bits, g, l, h, d_out, d_in, r)


def lb_gemv(x: torch.Tensor, lw: LittleBitWeight, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [d_out] fp32 of the LittleBit linear at batch 1 (x [d_in] or [1, d_in] bf16).
    workspace: reusable uint8 device buffer, zeroed once at allocation."""
    _dev(x, torch.bfloat16, "x")
    if x.numel() != lw.d_in:
        raise ValueError(f"x has {x.numel()} elements, the linear takes {lw.d_in}")
    if out is None:
        out = torch.empty(lw.d_out, dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
        if out.numel() != lw.d_out:
            raise ValueError("out must hold d_out values")
    need = int(lib().qlinear_lb_workspace_bytes(lw.d_out, lw.d_in, lw.rank))
    if workspace is None or workspace.numel() < need:
        # zeroed once: its slab counters must start at zero (every call leaves them zero)
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device)
    d = lw.desc()
    _check(lib().qlinear_lb_gemv(ctypes.byref(d), _ptr(x), _ptr(out), _ptr(workspace), need, _stream()), "lb_gemv")
    return out


# ---------------------------------------------------------------- 4-bit containers (baseline)
@dataclass
class C4Weight:
    """A weight stored as 4-bit containers (codes as two's complement nibbles), with the
    same packed scale array as the native layout."""
    c4: torch.Tensor          # uint8 container bytes
    pscales: torch.Tensor     # bfloat16, packed scale array
    N: int
    K: int

    @property
    def nbytes(self) -> int:
        return self.c4.numel() + 2 * self.pscales.numel()


def c4_pack(codes: torch.Tensor, scales: torch.Tensor) -> C4Weight:
    _dev(codes, torch.int8, "codes")
    _dev(scales, torch.bfloat16, "scales")
    N, K = codes.shape
    if tuple(scales.shape) != (N, K // GROUP):
        raise ValueError("scales must be [N, K/128]")
    size = int(lib().qlinear_c4_bytes(N, K))
    if size <= 0:
        raise ValueError(f"invalid shape {N}x{K}")
    c4 = torch.empty(size, dtype=torch.uint8, device=codes.device)
    _check(lib().qlinear_c4_pack(N, K, _ptr(codes), _ptr(c4), _stream()), "c4_pack")
    ps = torch.empty(packed_scales_len(N, K), dtype=torch.bfloat16, device=codes.device)
    _check(lib().qlinear_pack_scales(N, K, _ptr(scales), _ptr(ps), _stream()), "pack_scales")
    return C4Weight(c4, ps, N, K)


def c4_unpack(cw: C4Weight) -> torch.Tensor:
    codes = torch.empty((cw.N, cw.K), dtype=torch.int8, device=cw.c4.device)
    _check(lib().qlinear_c4_unpack(cw.N, cw.K, _ptr(cw.c4), _ptr(codes), _stream()), "c4_unpack")
    return codes


def c4_to_packed(cw: C4Weight, grid) -> PackedWeight:
    """Convert a container checkpoint to the native packed layout (codes must fit the grid)."""
    g, bg, bo, size = _grid_tables(cw.N, cw.K, grid, cw.c4.device)
    packed = torch.empty(size, dtype=torch.uint8, device=cw.c4.device)
    _check(lib().qlinear_c4_to_packed(cw.N, cw.K, g, _ptr(bg), _ptr(bo), _ptr(cw.c4), _ptr(packed), _stream()),
           "c4_to_packed")
    return PackedWeight(packed, cw.pscales, cw.N, cw.K, g, bg, bo)


def c4_gemv(x: torch.Tensor, cw: C4Weight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [1, N] fp32 = x [1, K] bf16 times the container weight transposed (batch 1)."""
    x, M, out = _xy(x, cw, out)
    _check(lib().qlinear_c4_gemv(M, cw.N, cw.K, _ptr(cw.c4), _ptr(cw.pscales), _ptr(x), _ptr(out), _stream()),
           "c4_gemv")
    return out


# ---------------------------------------------------------------- products
def _xy(x: torch.Tensor, pw: PackedWeight, out: Optional[torch.Tensor]):
    _dev(x, torch.bfloat16, "x")
    if x.dim() == 1:
        x = x.view(1, -1)
    M, K = x.shape
    if K != pw.K:
        raise ValueError(f"x has K={K}, weight has K={pw.K}")
    if out is None:
        out = torch.empty((M, pw.N), dtype=torch.float32, device=x.device)
    else:
        _dev(out, torch.float32, "out")
        if tuple(out.shape) != (M, pw.N):
            raise ValueError("out must be [M, N]")
    return x, M, out


def gemv(x: torch.Tensor, pw: PackedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] bf16 times the packed weight transposed, M <= 16."""
    x, M, out = _xy(x, pw, out)
    _check(lib().qlinear_gemv(M, pw.N, pw.K, pw.grid, _ptr(pw.blk_grid), _ptr(pw.blk_off), _ptr(pw.packed),
                              _ptr(pw.pscales), _ptr(x), _ptr(out), _stream()), "gemv")
    return out


def gemm(x: torch.Tensor, pw: PackedWeight, out: Optional[torch.Tensor] = None,
         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M, N] fp32 = x [M, K] bf16 times the packed weight transposed (MFMA path)."""
    x, M, out = _xy(x, pw, out)
    need = int(lib().qlinear_gemm_workspace_bytes(M, pw.N, pw.K))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(lib().qlinear_gemm(M, pw.N, pw.K, pw.grid, _ptr(pw.blk_grid), _ptr(pw.blk_off), _ptr(pw.packed),
                              _ptr(pw.pscales), _ptr(x), _ptr(out), _ptr(workspace), need, _stream()), "gemm")
    return out


def read_probe(buf, out):
    """out (256 int32 words) ^= the per-lane-position XOR of buf's 1 KB blocks (uint8 device tensor)."""
    _dev(buf, torch.uint8, "buf")
    _dev(out, torch.int32, "out")
    if out.numel() != 256:
        raise ValueError("out needs 256 words")
    _check(lib().qlinear_read_probe(_ptr(buf), buf.numel(), _ptr(out), _stream()), "read_probe")


def wave_slots(M=1):
    """Waves of a persistent grouped launch at batch size M on the current device."""
    n = lib().qlinear_grouped_wave_slots(M)
    if n < 0:
        _check(1, "grouped_wave_slots")
    return int(n)


class GroupedGemv:
    """One persistent launch over many independent (x, W, y) products with the same M."""

    def __init__(self, items, split=None, noalloc=False):
        """items: list of (PackedWeight or C4Weight, x [M,K] bf16, y [M,N] fp32); all of one kind.

        split: None (one task per 64-row slab), "auto" (cut the slabs' input into parts until
        the launch has half as many tasks as the device has wave slots, where rows allow: the
        best measured point for the per-layer launches of the 8B pass at M = 1 and 4),
        an int (that many parts for every item) or a list of ints (parts per item; 0 = auto).

        noalloc: run through qlinear_gemv_grouped_noalloc, whose scheduler and split-K state
        live in the library's static device array (no state tensor is allocated here)."""
        if not items:
            raise ValueError("no items")
        self.items = items
        self.M = items[0][1].shape[0] if items[0][1].dim() == 2 else 1
        self.containers = isinstance(items[0][0], C4Weight)
        if isinstance(split, (list, tuple)):
            if len(split) != len(items):
                raise ValueError("split: one entry per item")
            parts = [int(v) for v in split]
        elif isinstance(split, int) and not isinstance(split, bool):
            parts = [split] * len(items)
        elif split in (None, "auto"):
            parts = [0] * len(items)
        else:
            raise ValueError(f"split: {split!r}")
        arr = (ql_gemv_desc * len(items))()
        # heaviest slabs first (prepare then orders by task length, stably):
        # the launch ends on the cheapest tasks, which shortens its tail
        order = sorted(range(len(items)), key=lambda j: -items[j][0].nbytes / ((items[j][0].N + 63) // 64))
        for i, j in enumerate(order):
            pw, x, y = items[j]
            if isinstance(pw, C4Weight) != self.containers:
                raise ValueError("a grouped launch takes either containers or packed weights, not both")
            _dev(x, torch.bfloat16, "x")
            _dev(y, torch.float32, "y")
            m = x.shape[0] if x.dim() == 2 else 1
            if m != self.M or x.shape[-1] != pw.K or y.numel() != m * pw.N:
                raise ValueError(f"item {i}: shapes do not match")
            if self.containers:
                arr[i] = ql_gemv_desc(pw.c4.data_ptr(), pw.pscales.data_ptr(), None, None, x.data_ptr(),
                                      y.data_ptr(), pw.N, pw.K, GRID_C4, 0, parts[j], 0, 0)
            else:
                arr[i] = ql_gemv_desc(pw.packed.data_ptr(), pw.pscales.data_ptr(),
                                      pw.blk_grid.data_ptr() if pw.blk_grid is not None else None,
                                      pw.blk_off.data_ptr() if pw.blk_off is not None else None,
                                      x.data_ptr(), y.data_ptr(), pw.N, pw.K, pw.grid, 0, parts[j], 0, 0)
        if split is None:
            total = lib().qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(items))
            words = QL_SCHED_WORDS
        else:
            min_tasks = wave_slots(self.M) // 2 if any(v == 0 for v in parts) else 0
            w = ctypes.c_int64(0)
            total = lib().qlinear_grouped_prepare_split(ctypes.cast(arr, ctypes.c_void_p), len(items), min_tasks,
                                                        ctypes.byref(w))
            words = int(w.value)
        if total < 0:
            _check(1, "grouped_prepare")
        self.total = int(total)
        self.kparts = [int(arr[i].kparts) for i in range(len(items))]  # in launch order
        self.plan = [{"N": int(d.N), "K": int(d.K), "kparts": int(d.kparts), "ws_begin": int(d.ws_begin),
                      "slab_begin": int(d.slab_begin)} for d in arr]
        raw = bytes(memoryview(arr))
        self.count = len(items)
        self.descs = torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(items[0][1].device)
        self.state_words = words
        self.noalloc = bool(noalloc)
        if self.noalloc and (self.containers or words > QL_NOALLOC_STATE_WORDS):
            raise ValueError("noalloc launches take native grids and at most QL_NOALLOC_STATE_WORDS of state")
        # task counters and split state: zero once here, counters left zero by every completed launch
        self.sched = None if self.noalloc else torch.zeros(words, dtype=torch.int32, device=items[0][1].device)

    def run(self):
        if self.noalloc:
            _check(lib().qlinear_gemv_grouped_noalloc(_ptr(self.descs), self.count, self.total, self.M,
                                                      self.state_words, _stream()), "gemv_grouped_noalloc")
            return
        fn = lib().qlinear_c4_gemv_grouped if self.containers else lib().qlinear_gemv_grouped
        _check(fn(_ptr(self.descs), self.count, self.total, self.M, _ptr(self.sched), _stream()), "gemv_grouped")


class GroupedGemm:
    """One persistent large-tile GEMM launch (plus one reduction launch when K is split) over many
    independent (x, W, y) products at one M >= 16: qlinear_gemm_grouped."""

    def __init__(self, items):
        """items: list of (PackedWeight, x [M, K] bf16, y [M, N] fp32), all with the same M."""
        if not items:
            raise ValueError("no items")
        self.items = items
        self.M = items[0][1].shape[0]
        arr = (ql_gemv_desc * len(items))()
        for i, (pw, x, y) in enumerate(items):
            _dev(x, torch.bfloat16, "x")
            _dev(y, torch.float32, "y")
            if x.dim() != 2 or x.shape[0] != self.M or x.shape[1] != pw.K or y.numel() != self.M * pw.N:
                raise ValueError(f"item {i}: shapes do not match")
            arr[i] = ql_gemv_desc(pw.packed.data_ptr(), pw.pscales.data_ptr(),
                                  pw.blk_grid.data_ptr() if pw.blk_grid is not None else None,
                                  pw.blk_off.data_ptr() if pw.blk_off is not None else None,
                                  x.data_ptr(), y.data_ptr(), pw.N, pw.K, pw.grid, 0, 0, 0, 0)
        wsb = ctypes.c_int64(0)
        total = lib().qlinear_gemm_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(items), self.M,
                                                   ctypes.byref(wsb))
        if total < 0:
            _check(1, "gemm_grouped_prepare")
        self.total = int(total)
        self.count = len(items)
        self.plan = [{"N": int(d.N), "K": int(d.K), "splits": int(d.kparts), "first_task": int(d.slab_begin),
                      "ws_begin": int(d.ws_begin)} for d in arr]
        self.descs = torch.frombuffer(bytearray(bytes(memoryview(arr))), dtype=torch.uint8).to(items[0][1].device)
        self.ws_bytes = int(wsb.value)
        self.ws = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=items[0][1].device)

    def run(self):
        _check(lib().qlinear_gemm_grouped(_ptr(self.descs), self.count, self.total, self.M, _ptr(self.ws),
                                          self.ws_bytes, _stream()), "gemm_grouped")
