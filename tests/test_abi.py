"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments before touching the GPU (CPU only: no compute call reaches a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

from decode_gemv_thinkbit_amd import qlinear as ql

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "qlinear.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qlinear_\w+)\s*\(", src)))


def test_all_declared_symbols_exported():
    L = ql.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n


def test_sizes():
    assert ql.row_bytes(ql.GRID_T, 4096) == 832
    assert ql.row_bytes(ql.GRID_I2, 4096) == 1024
    assert ql.row_bytes(ql.GRID_I3, 4096) == 1536
    assert ql.row_bytes(ql.GRID_T, 100) == 0  # K not a multiple of 128
    assert ql.row_bytes(7, 128) == 0
    assert ql.lib().qlinear_packed_bytes(130, 256, ql.GRID_I2) == 3 * 64 * 64
    assert ql.packed_scales_len(70, 1280) == 2 * 2 * 64 * 8
    off = ql.block_offsets(300, 384, [0, 2, 1])
    assert list(off) == [0, 128 * 80, 128 * 80 + 128 * 144, 128 * 80 + 128 * 144 + 64 * 96]  # T row 80 B at K=384
    assert ql.lib().qlinear_version() == 2


def test_sizes_match_oracle(ora):
    for K in (128, 640, 1280, 4096, 5120, 12288, 17408):
        for g in (0, 1, 2):
            assert ql.row_bytes(g, K) == ora.row_bytes(g, K)
    t = np.array([2, 0, 1, 1, 0], np.int8)
    assert np.array_equal(ql.block_offsets(600, 2048, t), ora.block_offsets(600, 2048, t))


FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails validation first
MISALIGNED = ctypes.c_void_p(0x10008)


def status_and_msg(rc):
    return rc, ql.lib().qlinear_last_error().decode()


def test_gemv_argument_errors():
    L = ql.lib()
    args = lambda M, N, K, grid, p=FAKE: (M, N, K, grid, None, None, p, FAKE, FAKE, FAKE, None)
    rc, msg = status_and_msg(L.qlinear_gemv(*args(0, 64, 128, 0)))
    assert rc == 1 and "M" in msg
    rc, msg = status_and_msg(L.qlinear_gemv(*args(17, 64, 128, 0)))
    assert rc == 1
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 64, 100, 0)))
    assert rc == 1 and "multiple of 128" in msg
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 0, 128, 0)))
    assert rc == 1
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 64, 128, 5)))
    assert rc == 1 and "grid" in msg
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 64, 128, 3)))  # mixed without tables
    assert rc == 1 and "blk_grid" in msg
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 64, 128, 0, p=None)))
    assert rc == 1 and "null" in msg
    rc, msg = status_and_msg(L.qlinear_gemv(*args(1, 64, 128, 0, p=MISALIGNED)))
    assert rc == 1 and "aligned" in msg


def test_other_argument_errors():
    L = ql.lib()
    assert L.qlinear_gemm(0, 64, 128, 0, None, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == 1
    assert L.qlinear_quantize(4, 100, 0, None, FAKE, FAKE, FAKE, None) == 1
    assert L.qlinear_pack(4, 128, 3, None, None, FAKE, None, FAKE, None, None) == 1
    # scales without a packed scale array (or the reverse) is an argument error
    assert L.qlinear_pack(4, 128, 0, None, None, FAKE, FAKE, FAKE, None, None) == 1
    assert L.qlinear_pack(4, 128, 0, None, None, FAKE, None, FAKE, FAKE, None) == 1
    assert L.qlinear_unpack(4, 128, 9, None, None, FAKE, FAKE, None) == 1
    assert L.qlinear_dequant(4, 128, 0, None, None, None, FAKE, 0, FAKE, None) == 1
    assert L.qlinear_gemv_grouped(FAKE, 0, 10, 1, FAKE, None) == 1
    assert L.qlinear_gemv_grouped(FAKE, 2, 10, 17, FAKE, None) == 1  # batch above 16
    assert L.qlinear_gemv_grouped(FAKE, 2, 10, 0, FAKE, None) == 1
    assert L.qlinear_gemv_grouped(FAKE, 2, 10, 1, None, None) == 1  # no scheduler state
    assert L.qlinear_gemv_grouped(FAKE, 2, 10, 1, MISALIGNED, None) == 1
    bad = np.array([0, 7], np.int8)
    with pytest.raises(ql.QLinearError):
        ql.block_offsets(200, 128, bad)


def test_binding_rejects_host_tensors():
    import torch
    pw = ql.PackedWeight(torch.zeros(16, dtype=torch.uint8), torch.zeros(8, dtype=torch.bfloat16), 1, 128, 0)
    with pytest.raises(ValueError):
        ql.gemv(torch.zeros(1, 128, dtype=torch.bfloat16), pw)


def test_grouped_prepare_orders_longest_rows_first():
    """prepare sorts entries by K (largest first, stable) and numbers their slabs in that order."""
    L = ql.lib()
    shapes = [(100, 4096, 0), (64, 12288, 1), (300, 4096, 2), (1, 128, 0), (130, 12288, 0)]
    arr = (ql.ql_gemv_desc * len(shapes))()
    for i, (N, K, g) in enumerate(shapes):
        arr[i] = ql.ql_gemv_desc(FAKE, FAKE, None, None, FAKE, FAKE, N, K, g, -1)
        arr[i].slab_begin = i  # tag, overwritten by prepare
    tags = {(N, K, g): i for i, (N, K, g) in enumerate(shapes)}
    total = L.qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(shapes))
    got = [(d.N, d.K, d.grid) for d in arr]
    assert got == sorted(shapes, key=lambda s: (-s[1], tags[s]))
    begins = [d.slab_begin for d in arr]
    assert begins == list(np.cumsum([0] + [(n + 63) // 64 for n, _, _ in got])[:-1])
    assert total == sum((n + 63) // 64 for n, _, _ in shapes)


def test_container_sizes_and_argument_errors():
    L = ql.lib()
    assert L.qlinear_c4_bytes(130, 256) == 3 * 64 * 128
    assert L.qlinear_c4_bytes(130, 100) == 0
    p = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    assert L.qlinear_c4_gemv(2, 64, 128, p, p, p, p, None) == 2      # batch 1 only
    assert L.qlinear_c4_gemv(1, 64, 100, p, p, p, p, None) == 1      # K % 128
    assert L.qlinear_c4_gemv(1, 64, 128, None, p, p, p, None) == 1   # null container
    assert L.qlinear_c4_pack(64, 128, ctypes.c_void_p(8), p, None) == 1  # misaligned
    assert L.qlinear_c4_to_packed(64, 128, 4, None, None, p, p, None) == 1  # 4 is not a ThinkBit grid
    assert L.qlinear_c4_gemv_grouped(p, 1, 1, 4, p, None) == 2
    assert L.qlinear_c4_gemv_grouped(p, 1, 1, 1, None, None) == 1
    assert L.qlinear_pack(64, 128, ql.GRID_C4, None, None, p, None, p, None, None) == 1  # native rejects containers


def test_grouped_prepare_rejects_mixed_container_lists():
    L = ql.lib()
    arr = (ql.ql_gemv_desc * 2)()
    arr[0] = ql.ql_gemv_desc(16, 32, None, None, 48, 64, 64, 128, ql.GRID_C4, 0)
    arr[1] = ql.ql_gemv_desc(16, 32, None, None, 48, 64, 64, 256, ql.GRID_I2, 0)
    assert L.qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), 2) == -1
    assert b"mix" in L.qlinear_last_error()
    arr[1] = ql.ql_gemv_desc(16, 32, None, None, 48, 64, 64, 256, ql.GRID_C4, 0)
    assert L.qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), 2) == 2
    assert arr[0].K == 256 and arr[0].slab_begin == 0 and arr[1].slab_begin == 1


def _descs(shapes, parts):
    arr = (ql.ql_gemv_desc * len(shapes))()
    for i, ((N, K, g), p) in enumerate(zip(shapes, parts)):
        arr[i] = ql.ql_gemv_desc(FAKE, FAKE, None, None, FAKE, FAKE, N, K, g, -1, p, 7, 99)
    return arr


def test_grouped_prepare_split_plans_parts_and_state():
    """Split plan: parts per slab (forced, clamped to the row's 640-input periods, or enough
    for min_tasks), task order by part length, task numbering, and the state layout: the
    queue words, then per split entry one 32-word counter line per slab and 1024 words of
    partial sums per (slab, part)."""
    L = ql.lib()
    shapes = [(4096, 4096, 0), (1024, 4096, 2), (100, 128, 1), (4096, 12288, 0), (130, 5120, 1)]
    arr = _descs(shapes, [0, 3, 0, 0, 50])
    words = ctypes.c_int64(-1)
    slabs = [(n + 63) // 64 for n, _, _ in shapes]
    min_tasks = 4096
    total = L.qlinear_grouped_prepare_split(ctypes.cast(arr, ctypes.c_void_p), len(shapes), min_tasks,
                                            ctypes.byref(words))
    need = -(-min_tasks // sum(slabs))
    periods = {K: -(-K // 640) for _, K, _ in shapes}
    cap = ql.QL_MAX_KPARTS
    want = {(4096, 4096, 0): min(need, 7, cap), (1024, 4096, 2): 3, (100, 128, 1): 1,
            (4096, 12288, 0): min(need, 20, cap), (130, 5120, 1): 8}
    got = {(d.N, d.K, d.grid): d.kparts for d in arr}
    assert got == want
    assert all(1 <= d.kparts <= min(periods[d.K], cap) for d in arr)
    # longest parts first (K / kparts), stable
    keys = [d.K / d.kparts for d in arr]
    assert keys == sorted(keys, reverse=True)
    ntask = [((d.N + 63) // 64) * d.kparts for d in arr]
    assert [d.slab_begin for d in arr] == list(np.cumsum([0] + ntask)[:-1])
    assert total == sum(ntask)
    w = (ql.QL_SCHED_WORDS + 63) // 64 * 64
    for d in arr:
        assert d.reserved == 0
        if d.kparts == 1:
            assert d.ws_begin == 0
            continue
        ns = (d.N + 63) // 64
        assert d.ws_begin == w
        w += ns * 32 + ns * d.kparts * 1024
    assert words.value == w


def test_grouped_prepare_split_without_split_matches_prepare():
    L = ql.lib()
    shapes = [(100, 4096, 0), (64, 12288, 1), (300, 4096, 2), (1, 128, 0)]
    a, b = _descs(shapes, [0] * 4), _descs(shapes, [0] * 4)
    words = ctypes.c_int64(-1)
    ta = L.qlinear_grouped_prepare(ctypes.cast(a, ctypes.c_void_p), 4)
    tb = L.qlinear_grouped_prepare_split(ctypes.cast(b, ctypes.c_void_p), 4, 0, ctypes.byref(words))
    assert ta == tb == sum((n + 63) // 64 for n, _, _ in shapes)
    assert words.value == ql.QL_SCHED_WORDS
    assert bytes(memoryview(a)) == bytes(memoryview(b))
    assert all(d.kparts == 1 and d.ws_begin == 0 for d in a)
    # plain prepare ignores requested parts
    c = _descs(shapes, [5] * 4)
    assert L.qlinear_grouped_prepare(ctypes.cast(c, ctypes.c_void_p), 4) == ta
    assert all(d.kparts == 1 for d in c)


def test_grouped_prepare_split_rejects_bad_parts_and_split_containers():
    L = ql.lib()
    words = ctypes.c_int64(-1)
    arr = _descs([(64, 256, 0)], [-1])
    assert L.qlinear_grouped_prepare_split(ctypes.cast(arr, ctypes.c_void_p), 1, 0, ctypes.byref(words)) == -1
    arr = _descs([(64, 1280, ql.GRID_C4), (64, 1280, ql.GRID_C4)], [2, 0])
    assert L.qlinear_grouped_prepare_split(ctypes.cast(arr, ctypes.c_void_p), 2, 0, ctypes.byref(words)) == -1
    assert b"not split" in L.qlinear_last_error()
    arr = _descs([(64, 1280, ql.GRID_C4), (64, 1280, ql.GRID_C4)], [0, 0])
    assert L.qlinear_grouped_prepare_split(ctypes.cast(arr, ctypes.c_void_p), 2, 10 ** 6, ctypes.byref(words)) == 2
    assert all(d.kparts == 1 for d in arr) and words.value == ql.QL_SCHED_WORDS


def test_split_periods_tile_every_row():
    """The device's part ranges, p0 = part * P // parts .. (part + 1) * P // parts, tile
    [0, P) with no empty part for every parts <= P."""
    for P in range(1, 40):
        for parts in range(1, P + 1):
            r = [(q * P // parts, (q + 1) * P // parts) for q in range(parts)]
            assert r[0][0] == 0 and r[-1][1] == P
            assert all(a < b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(parts - 1))


def test_wave_slots_query():
    L = ql.lib()
    assert L.qlinear_grouped_wave_slots(0) == -1 and L.qlinear_grouped_wave_slots(17) == -1
    n1, n4, n16 = (L.qlinear_grouped_wave_slots(m) for m in (1, 4, 16))
    # batch 1 and 2..4 tokens: 2 workgroups x 8 waves per CU; 5..16 tokens: 2 x 6
    assert n1 > 0 and n1 == n4 and n1 % 16 == 0 and n16 > 0 and n16 % 12 == 0


def test_read_probe_argument_errors():
    L = ql.lib()
    p = ctypes.c_void_p(0x10000)
    assert L.qlinear_read_probe(p, 0, p, None) == 1
    assert L.qlinear_read_probe(p, 1000, p, None) == 1          # not a multiple of 1024
    assert L.qlinear_read_probe(p, 1 << 32, p, None) == 1       # offsets are 32-bit
    assert L.qlinear_read_probe(None, 1024, p, None) == 1
    assert L.qlinear_read_probe(p, 1024, ctypes.c_void_p(0x10004), None) == 1  # misaligned out


def test_grouped_prepare_rejects_rows_beyond_the_batched_range():
    """The GEMV kernel addresses all tokens' activations in one 32-bit range: K above 2^26
    is refused before any launch."""
    L = ql.lib()
    arr = _descs([(64, (1 << 26) + 128, 0)], [1])
    assert L.qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), 1) == -1
    assert b"K=" in L.qlinear_last_error()
    arr = _descs([(64, 1 << 26, 0)], [1])
    assert L.qlinear_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), 1) == 1


def test_gemm_grouped_prepare_plan_and_errors():
    """Host plan of the grouped GEMM: entries longest-first with consecutive task ranges, the
    workspace covering every split entry's partials, and bad arguments rejected."""
    L = ql.lib()
    shapes = [(4096, 4096), (1024, 4096), (4096, 12288), (12288, 4096)]

    def arr_of():
        arr = (ql.ql_gemv_desc * len(shapes))()
        for i, (N, K) in enumerate(shapes):
            base = 0x100000 * (i + 1)
            arr[i] = ql.ql_gemv_desc(base, base + 0x1000, None, None, base + 0x2000, base + 0x3000, N, K, 0, 0, 0, 0, 0)
        return arr

    for M in (16, 64, 256, 512):
        arr = arr_of()
        ws = ctypes.c_int64(-1)
        total = L.qlinear_gemm_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(shapes), M, ctypes.byref(ws))
        assert total > 0
        mt = (M + 64 * (1 if M <= 64 else 2 if M <= 128 else 4) - 1) // (64 * (1 if M <= 64 else 2 if M <= 128 else 4))
        first, need, prev = 0, 0, None
        for d in arr:
            assert d.slab_begin == first and 1 <= d.kparts <= 16
            stages = (d.K // 64 + d.kparts - 1) // d.kparts
            assert prev is None or stages <= prev + 1  # longest tasks first (stage counts)
            prev = stages
            first += ((d.N + 255) // 256) * mt * d.kparts
            if d.kparts > 1:
                assert d.ws_begin >= need and d.ws_begin % 64 == 0
                need = d.ws_begin + d.kparts * M * d.N
        assert first == total and ws.value >= 4 * need
    arr = arr_of()
    assert L.qlinear_gemm_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(shapes), 8, None) == -1
    assert L.qlinear_gemm_grouped_prepare(None, 0, 64, None) == -1
    arr[1].K = 100  # not a multiple of 128
    assert L.qlinear_gemm_grouped_prepare(ctypes.cast(arr, ctypes.c_void_p), len(shapes), 64, None) == -1
    assert L.qlinear_gemm_grouped(None, 1, 1, 64, None, 0, None) != 0
