"""Host-side checks of the C ABI: the library loads, exports what include/squad.h
declares, rejects bad arguments before touching the device, and its address maps
are the oracle's window partition.  No GPU needed."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sub_quadratic_windowed_amd import _lib
import sub_quadratic_windowed_amd as sq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "squad.h")

OK, INVALID, SHAPE, UNSUP, ALIAS, ALIGN, WORKSPACE, HIP, SCRATCH = range(9)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(squad_[a-z_0-9]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    lib = _lib.lib()
    declared = header_functions()
    assert len(declared) >= 10, declared
    assert sorted(_lib.EXPORTS) == declared
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    lib = _lib.lib()
    for s in range(9):
        assert lib.squad_status_string(s).decode() != "unknown status"
    assert lib.squad_status_string(99).decode() == "unknown status"


def test_workspace_size():
    assert sq.squad_attn_workspace_size((64, 48, 80), (4, 12, 10), 24, 1, 128, 1) == 245760 * 24 * 128 * 2
    assert sq.squad_attn_workspace_size((4, 8, 8), (1, 4, 4), 2, 1, 64, 0) == 256 * 2 * 64 * 4
    # a cut tiling: 2 x 2 x 2 windows of 48 cells, absent cells included
    assert sq.squad_attn_workspace_size((4, 8, 8), (3, 4, 4), 2, 1, 64, 0) == 8 * 48 * 2 * 64 * 4
    assert sq.squad_attn_workspace_size((4, 8, 8), (5, 4, 4), 2, 1, 64, 0) == 0    # tile larger than the grid
    # cut tilings with more than 512 windows run in bf16 too
    assert sq.squad_attn_workspace_size((33, 32, 32), (2, 1, 1), 1, 1, 64, 1) == 17 * 32 * 32 * 2 * 64 * 2
    assert sq.squad_attn_workspace_size((33, 32, 32), (2, 1, 1), 1, 1, 64, 0) == 17 * 32 * 32 * 2 * 64 * 4
    assert sq.squad_attn_workspace_size((4, 8, 8), (1, 4, 4), 2, 1, 96, 1) == 0


# fake, never-dereferenced device addresses: argument checks must fire first
A = 0x10000000
B = 0x20000000
C = 0x30000000
O = 0x40000000
WS = 0x50000000


def fwd(q=A, k=B, v=C, grid=(4, 8, 8), tile=(1, 4, 4), heads=2, out=O, batch=1, d=64, dtype=1,
        scale=0.0, ws=WS, ws_bytes=1 << 30):
    return _lib.lib().squad_attn_forward(
        ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), _lib.int3(grid), _lib.int3(tile), heads,
        ctypes.c_void_p(out), batch, d, dtype, ctypes.c_float(scale), ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(out=0), INVALID), (dict(heads=0), INVALID), (dict(batch=-1), INVALID),
    (dict(grid=(4, 0, 8)), INVALID), (dict(tile=(1, 4, -4)), INVALID),
    (dict(tile=(5, 4, 4)), SHAPE), (dict(tile=(1, 9, 4)), SHAPE), (dict(grid=(1 << 11, 1 << 11, 1 << 10)), SHAPE),
    (dict(tile=(3, 4, 4), ws_bytes=8 * 48 * 2 * 64 * 2 - 1), WORKSPACE),
    (dict(d=96), UNSUP), (dict(d=256), UNSUP), (dict(dtype=2), UNSUP),
    (dict(q=A + 8), ALIGN), (dict(out=O + 4), ALIGN), (dict(ws=WS + 2), ALIGN),
    (dict(out=A), ALIAS), (dict(out=B + 64), ALIAS), (dict(ws=C), ALIAS), (dict(ws=O), ALIAS),
    (dict(ws=0), WORKSPACE), (dict(ws_bytes=256 * 2 * 64 * 2 - 1), WORKSPACE),
    (dict(scale=float("nan")), INVALID),
])
def test_forward_rejects_bad_arguments(kw, status):
    assert fwd(**kw) == status


def fwd_noalloc(q=A, k=B, v=C, grid=(4, 8, 8), tile=(1, 4, 4), heads=2, out=O, batch=1, d=64, dtype=1,
                scale=0.0):
    return _lib.lib().squad_attn_forward_noalloc(
        ctypes.c_void_p(q), ctypes.c_void_p(k), ctypes.c_void_p(v), _lib.int3(grid), _lib.int3(tile), heads,
        ctypes.c_void_p(out), batch, d, dtype, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), INVALID), (dict(out=0), INVALID), (dict(heads=0), INVALID), (dict(tile=(5, 4, 4)), SHAPE),
    (dict(d=96), UNSUP), (dict(dtype=2), UNSUP), (dict(q=A + 8), ALIGN), (dict(out=B + 64), ALIAS),
    (dict(scale=float("nan")), INVALID),
    # one (batch, head)'s local output past the 64 MiB scratch: 266,240 cells x 128 x 2 bytes
    (dict(grid=(64, 64, 65), tile=(4, 8, 5), heads=1, d=128), SCRATCH),
    # fp32: 262,144 cells x 128 x 4 bytes = 128 MiB
    (dict(grid=(64, 64, 64), tile=(4, 8, 8), heads=1, d=128, dtype=0), SCRATCH),
])
def test_noalloc_rejects_bad_arguments(kw, status):
    """The checks run on the host before the scratch is looked up or anything is
    enqueued (no device here)."""
    assert fwd_noalloc(**kw) == status


def test_noalloc_scratch_limit_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define SQUAD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_other_entry_points_reject_bad_arguments():
    lib = _lib.lib()
    p = ctypes.c_void_p
    g, t = _lib.int3((4, 8, 8)), _lib.int3((1, 4, 4))
    for fn in (lib.squad_tile_gather, lib.squad_tile_scatter, lib.squad_window_to_group):
        assert fn(p(A), p(0), g, t, 2, 1, 64, 1, None) == INVALID
        assert fn(p(A), p(A), g, t, 2, 1, 64, 1, None) == ALIAS
        assert fn(p(A), p(B), g, _lib.int3((1, 3, 4)), 2, 1, 64, 1, None) == SHAPE
        assert fn(p(A), p(B + 2), g, t, 2, 1, 64, 1, None) == ALIGN
    for fn in (lib.squad_local_pass, lib.squad_global_pass):
        assert fn(p(A), p(B), p(C), g, t, 2, p(C), 1, 64, 1, ctypes.c_float(0), None) == ALIAS
        assert fn(p(A), p(B), p(C), g, t, 2, p(O), 1, 32, 1, ctypes.c_float(0), None) == UNSUP
    assert lib.squad_window_attn(p(A), p(B), p(C), p(O), 0, 16, 64, 1, ctypes.c_float(0), None) == INVALID
    assert lib.squad_window_attn(p(A), p(B), p(C), p(A), 4, 16, 64, 1, ctypes.c_float(0), None) == ALIAS
    assert lib.squad_dense_attn_forward(p(A), p(B), p(C), p(O), 1, 0, 2, 64, 1, ctypes.c_float(0), None) == INVALID
    assert lib.squad_dense_attn_forward(p(A), p(B), p(C), p(O), 1, 256, 2, 64, 7, ctypes.c_float(0), None) == UNSUP
    off = np.zeros(512, np.int64)
    ptr = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    assert lib.squad_debug_row_offsets(4, g, t, 2, 1, 64, ptr) == INVALID


# ---------------------------------------------------------------- address maps vs the oracle's partition

MAP_SHAPES = [((4, 8, 8), (1, 4, 4)), ((2, 4, 6), (2, 2, 3)), ((3, 2, 4), (1, 2, 2)), ((2, 3, 4), (1, 1, 1)),
              ((1, 4, 4), (1, 4, 4)), ((32, 24, 40), (2, 8, 10)), ((4, 6, 10), (4, 6, 10))]


@pytest.mark.parametrize("grid,tile", MAP_SHAPES)
@pytest.mark.parametrize("batch,heads,d", [(1, 2, 64), (2, 3, 128)])
def test_row_maps_are_the_window_partition(grid, tile, batch, heads, d):
    idx = oracle.window_index(grid, tile)                 # [G, Wn] token of (window, offset)
    G, Wn = idx.shape
    n = G * Wn
    b = np.arange(batch)[:, None, None, None]
    h = np.arange(heads)[None, :, None, None]
    # which = 0: (b, h, g, p) -> token order offset of token idx[g, p]
    want0 = ((b * n + idx[None, None]) * heads + h) * d
    got0 = sq.squad_debug_row_offsets(0, grid, tile, heads, batch, d).reshape(batch, heads, G, Wn)
    assert np.array_equal(got0, want0)
    # which = 1: (b, h, p, g) -> token idx[g, p]
    want1 = ((b * n + idx.T[None, None]) * heads + h) * d
    got1 = sq.squad_debug_row_offsets(1, grid, tile, heads, batch, d).reshape(batch, heads, Wn, G)
    assert np.array_equal(got1, want1)
    # which = 2 / 3: group-major [B, heads, Wn, G, d]
    gi = np.arange(G)[:, None]
    pi = np.arange(Wn)[None, :]
    want2 = (((b * heads + h) * Wn + pi[None, None]) * G + gi[None, None]) * d
    got2 = sq.squad_debug_row_offsets(2, grid, tile, heads, batch, d).reshape(batch, heads, G, Wn)
    assert np.array_equal(got2, want2)
    got3 = sq.squad_debug_row_offsets(3, grid, tile, heads, batch, d).reshape(batch, heads, Wn, G)
    assert np.array_equal(got3, np.swapaxes(want2, 2, 3))
    # every map is a bijection onto the rows of its tensor
    for got in (got0, got1, got2, got3):
        assert np.array_equal(np.sort(got.ravel()), np.arange(batch * heads * n) * d)


def test_row_maps_at_full_size():
    """The largest configuration: both token maps cover every row exactly once."""
    grid, tile, heads = (64, 48, 80), (4, 12, 10), 24
    n = 64 * 48 * 80
    for which in (0, 1):
        got = sq.squad_debug_row_offsets(which, grid, tile, heads, 1, 128)
        assert got.size == n * heads
        assert np.array_equal(np.sort(got), np.arange(n * heads) * 128)
    idx = oracle.window_index(grid, tile)
    got0 = sq.squad_debug_row_offsets(0, grid, tile, heads, 1, 128).reshape(heads, *idx.shape)
    assert np.array_equal(got0[5], (idx * heads + 5) * 128)


def test_wide_row_maps_past_2_to_the_31():
    """Tensors of 2^31 elements or more per batch element take wide maps (row offsets
    in head rows): 128^3 tokens x 8 heads x 128 dims = 2^31.  The offsets the maps
    give, turned back into elements, are every row of each tensor exactly once, and
    the local pass's token map puts head h of window g, offset p at the oracle's
    token index (g, p)."""
    grid, tile, heads, d = (128, 128, 128), (8, 16, 16), 8, 128
    n = 128 ** 3
    assert n * heads * d == 1 << 31
    idx = oracle.window_index(grid, tile)             # [G, Wn] token indices
    got0 = sq.squad_debug_row_offsets(0, grid, tile, heads, 1, d)
    assert np.array_equal(np.sort(got0), np.arange(n * heads, dtype=np.int64) * d)
    got0 = got0.reshape(heads, *idx.shape)
    for h in (0, 5, 7):
        assert np.array_equal(got0[h], (idx.astype(np.int64) * heads + h) * d)
    del got0
    got1 = sq.squad_debug_row_offsets(1, grid, tile, heads, 1, d).reshape(heads, idx.shape[1], idx.shape[0])
    assert np.array_equal(got1[7], (idx.T.astype(np.int64) * heads + 7) * d)
    del got1
    for which in (2, 3):   # the workspace, group-major
        got = sq.squad_debug_row_offsets(which, grid, tile, heads, 1, d)
        assert np.array_equal(np.sort(got), np.arange(n * heads, dtype=np.int64) * d)


def test_wide_row_maps_on_a_cut_tiling():
    """A cut tiling past 2^31 elements (127 x 128 x 130 grid, 8 x 16 x 16 tiles:
    1,152 windows of 2,048 cells, 2,113,280 tokens, 8 heads x 128): the present
    rows of both token maps are every row of the tensor once; absent rows read -1."""
    grid, tile, heads, d = (127, 128, 130), (8, 16, 16), 8, 128
    n = 127 * 128 * 130
    cells = 16 * 8 * 9 * 2048
    assert cells * heads * d >= 1 << 31
    for which in (0, 1):
        got = sq.squad_debug_row_offsets(which, grid, tile, heads, 1, d)
        assert got.size == cells * heads
        present = got[got >= 0]
        assert (got == -1).sum() == (cells - n) * heads
        assert np.array_equal(np.sort(present), np.arange(n * heads, dtype=np.int64) * d)


def test_row_unit_limits():
    """Wide maps reach 2^32 - 2 head rows per batch element: 2^30 cells x 3 heads
    are accepted (workspace size above zero), x 4 heads (2^32 rows) are not."""
    g, t = (1024, 1024, 1024), (16, 32, 32)
    assert sq.squad_attn_workspace_size(g, t, 3, 1, 128, 1) == 3 * (1 << 30) * 128 * 2
    assert sq.squad_attn_workspace_size(g, t, 4, 1, 128, 1) == 0


def _device_count():
    try:
        import torch
        return torch.cuda.device_count()
    except Exception:  # pragma: no cover
        return 0


@pytest.mark.skipif(_device_count() > 0, reason="fake pointers must never reach a real device")
def test_valid_call_without_device_reports_hip_error():
    assert fwd() == HIP


# ---------------------------------------------------------------- tile planner (host-only)

def _plan_cost(grid, tile):
    wn = int(np.prod(tile))
    gp = int(np.prod([-(-g // t) for g, t in zip(grid, tile)]))
    return gp * wn * (wn + gp), gp * wn - int(np.prod(grid))


@pytest.mark.parametrize("grid", [(64, 48, 80), (32, 24, 40), (16, 16, 16), (4, 8, 8), (21, 45, 80),
                                  (7, 7, 7), (1, 1, 1), (5, 3, 1), (2, 1, 97)])
def test_plan_tile_is_the_cheapest_tiling(grid):
    """Brute force over every tile no larger than the grid: the planner's pick has
    the least product work, and the fewest absent cells among the cheapest."""
    tile = sq.squad_plan_tile(grid)
    assert all(1 <= t <= g for t, g in zip(tile, grid))
    tiles = [(a, b, c) for a in range(1, grid[0] + 1) for b in range(1, grid[1] + 1) for c in range(1, grid[2] + 1)]
    best = min(_plan_cost(grid, t) for t in tiles)
    assert _plan_cost(grid, tile) == best
    # among those, the most compact window: per axis, extent close to the window count
    skew = min(_skew(grid, t) for t in tiles if _plan_cost(grid, t) == best)
    assert _skew(grid, tile) <= skew + 1e-9


def _skew(grid, tile):
    return sum(np.log(t / -(-g // t)) ** 2 for g, t in zip(grid, tile))


def test_plan_tile_prefers_compact_windows():
    # equal work and no absent tokens: (8, 6, 10) has 8 x 8 x 8 windows, (4, 12, 10)
    # and (1, 6, 80) have the same sizes but stretched windows
    assert sq.squad_plan_tile((64, 48, 80)) == (8, 6, 10)
    assert sq.squad_plan_tile((16, 16, 16)) == (4, 4, 4)
    assert sq.squad_plan_tile((64, 32, 32)) == (8, 4, 8)


def test_plan_tile_near_sqrt_n():
    # whole tilings with W = G = sqrt(n) exist for these grids; the planner finds one
    for grid in [(16, 16, 16), (4, 8, 8), (1, 64, 64)]:
        tile = sq.squad_plan_tile(grid)
        n = int(np.prod(grid))
        assert int(np.prod(tile)) ** 2 == n and _plan_cost(grid, tile)[1] == 0


def _planner_grids():
    """Grids up to twice the high-resolution workload's 245,760 tokens: the
    configurations' grids, grids with no whole tiling near sqrt(n), and a seeded
    random sample."""
    grids = [(64, 48, 80), (128, 48, 80), (65, 65, 65), (127, 49, 79), (61, 67, 71), (97, 89, 53),
             (1, 491, 1000), (3, 401, 401), (78, 78, 78), (2, 1, 97)]
    rng = np.random.default_rng(11)
    while len(grids) < 60:
        g = tuple(int(x) for x in rng.integers(1, 161, size=3))
        if np.prod(g) <= 2 * 245760:
            grids.append(g)
    return grids


def test_planned_tiles_run_in_bf16():
    """Whatever tile the planner picks (whole or cut, any number of windows) is
    accepted by the bf16 forward and training calls at 24 heads of 128."""
    for grid in _planner_grids():
        tile = sq.squad_plan_tile(grid)
        for fn in (sq.squad_attn_workspace_size, sq.squad_attn_train_workspace_size):
            assert fn(grid, tile, 24, 1, 128, 1) > 0, (grid, tile, fn.__name__)
    assert sq.squad_plan_tile((65, 65, 65)) == (3, 13, 13)   # 550 windows of 507 cells


def test_plan_tile_rejects_bad_grids():
    lib = _lib.lib()
    out = (ctypes.c_int32 * 3)()
    assert lib.squad_plan_tile(_lib.int3((4, 0, 8)), out) == INVALID
    assert lib.squad_plan_tile(_lib.int3((1 << 11, 1 << 11, 1 << 10)), out) == SHAPE


# ---------------------------------------------------------------- cut tilings: the kernels' presence test

CUT_MAP_SHAPES = [((3, 5, 7), (2, 2, 3)), ((5, 12, 20), (2, 5, 6)), ((4, 8, 8), (3, 4, 4)),
                  ((2, 3, 4), (2, 3, 3)), ((7, 7, 7), (1, 2, 7)), ((33, 32, 32), (2, 1, 1))]


@pytest.mark.parametrize("grid,tile", CUT_MAP_SHAPES)
def test_cut_row_maps_are_the_padded_partition(grid, tile):
    """On a cut tiling the token maps, with the presence test the kernels use to skip
    absent rows, are the oracle's padded window partition: -1 exactly at absent
    cells, the token's row elsewhere; the workspace maps stay a bijection over all
    tile cells."""
    heads, batch, d = 2, 2, 64
    idx = oracle.padded_window_index(grid, tile)          # [G, Wn], -1 for absent cells
    G, Wn = idx.shape
    n = int(np.prod(grid))
    b = np.arange(batch)[:, None, None, None]
    h = np.arange(heads)[None, :, None, None]
    want0 = np.where(idx[None, None] >= 0, ((b * n + idx[None, None]) * heads + h) * d, -1)
    got0 = sq.squad_debug_row_offsets(0, grid, tile, heads, batch, d).reshape(batch, heads, G, Wn)
    assert np.array_equal(got0, want0)
    got1 = sq.squad_debug_row_offsets(1, grid, tile, heads, batch, d).reshape(batch, heads, Wn, G)
    assert np.array_equal(got1, np.swapaxes(want0, 2, 3))
    # row 0 of every unit is present (the kernels' clamp target for absent queries)
    assert (got0[:, :, :, 0] >= 0).all() and (got1[:, :, :, 0] >= 0).all()
    for which in (2, 3):
        got = sq.squad_debug_row_offsets(which, grid, tile, heads, batch, d)
        assert np.array_equal(np.sort(got), np.arange(batch * heads * G * Wn) * d)


def test_cut_tilings_at_the_half_pass_entry_points():
    lib = _lib.lib()
    p = ctypes.c_void_p
    t = _lib.int3((2, 3, 3))
    for fn in (lib.squad_local_pass, lib.squad_global_pass):
        # accepted up to the device call (fake pointers: HIP error without a device)
        if _device_count() == 0:
            assert fn(p(A), p(B), p(C), _lib.int3((3, 5, 7)), t, 2, p(O), 1, 64, 1, ctypes.c_float(0), None) == HIP
    for fn in (lib.squad_tile_gather, lib.squad_tile_scatter, lib.squad_window_to_group):
        assert fn(p(A), p(B), _lib.int3((3, 5, 7)), t, 2, 1, 64, 1, None) == SHAPE


# ---------------------------------------------------------------- k-level maps (host-only)

KPASS_SHAPES = [((4, 8, 8), [(1, 2, 2), (2, 4, 4)]), ((4, 4, 8), [(1, 2, 2), (2, 2, 4), (2, 4, 8)]),
                ((2, 8, 4), [(2, 2, 1), (2, 4, 2)]), ((64, 48, 80), [(4, 4, 4), (16, 16, 16)])]


@pytest.mark.parametrize("grid,tiles", KPASS_SHAPES)
def test_kpass_maps_are_the_level_partitions(grid, tiles):
    """Every level's six-digit map sends (unit, row) to the token the oracle's level
    index puts there (same row order; units may be numbered differently)."""
    heads, batch, d = 2, 1, 64
    n = int(np.prod(grid))
    for level in range(len(tiles) + 1):
        idx = oracle.kpass_level_index(grid, tiles, level)           # [U, L] tokens
        U, L = idx.shape
        got = sq.squad_debug_kpass_offsets(grid, tiles, level, heads, batch, d).reshape(batch, heads, U, L)
        for h in range(heads):
            tok = (got[0, h] - h * d) // (heads * d)
            assert ((got[0, h] - h * d) % (heads * d) == 0).all()
            # each unit is a unit of the oracle, rows in the same order
            assert np.array_equal(np.sort(tok[:, 0]), np.sort(idx[:, 0]))
            pos = {int(t): i for i, t in enumerate(idx[:, 0])}
            assert np.array_equal(tok, idx[[pos[int(t)] for t in tok[:, 0]]])
        if n > 10000:
            break


def test_kpass_argument_checks():
    lib = _lib.lib()
    p = ctypes.c_void_p
    ws = lambda g, t: sq.squad_kpass_workspace_size(g, t, 2, 1, 64, 1)
    assert ws((4, 8, 8), [(1, 2, 2), (2, 4, 4)]) == 2 * 256 * 2 * 64 * 2
    assert ws((4, 8, 8), [(1, 4, 4)]) == 256 * 2 * 64 * 2
    assert ws((4, 8, 8), [(1, 4, 4), (2, 2, 8)]) == 0                 # not nested
    assert ws((4, 8, 8), [(1, 2, 2)] * 8) == 0                         # more than 8 levels
    arr = (ctypes.c_int32 * 6)(1, 2, 2, 2, 4, 4)
    g = _lib.int3((4, 8, 8))
    call = lambda levels=3, d=64, out=O, w=WS, wb=1 << 30: lib.squad_kpass_forward(
        p(A), p(B), p(C), g, arr, levels, 2, p(out), 1, d, 1, ctypes.c_float(0), p(w), wb, None)
    assert call(levels=1) == INVALID
    assert call(d=96) == UNSUP
    assert call(out=A) == ALIAS
    assert call(w=0) == WORKSPACE
    assert call(wb=2 * 256 * 2 * 64 * 2 - 1) == WORKSPACE
    bad = (ctypes.c_int32 * 6)(1, 4, 4, 2, 2, 8)
    assert lib.squad_kpass_forward(p(A), p(B), p(C), g, bad, 3, 2, p(O), 1, 64, 1, ctypes.c_float(0), p(WS),
                                   1 << 30, None) == SHAPE
    if _device_count() == 0:
        assert call() == HIP


# ---------------------------------------------------------------- training and block entry points (host-only)

def test_training_entry_points_reject_bad_arguments():
    lib = _lib.lib()
    p = ctypes.c_void_p
    g, t = _lib.int3((4, 8, 8)), _lib.int3((1, 4, 4))
    need = sq.squad_attn_train_workspace_size((4, 8, 8), (1, 4, 4), 2, 1, 64, 1)
    # O1 (fp16), 4 per-row fp32 arrays (two passes' statistics and D), the local
    # output's gradient, and one inverse scale per head row of dq and of dk
    assert need == 256 * 2 * 64 * 2 * 2 + 4 * 256 * 2 * 4 + 2 * 256 * 2 * 4
    assert sq.squad_attn_train_workspace_size((4, 8, 8), (5, 4, 4), 2, 1, 64, 1) == 0
    D, K, V, OUT, DOUT = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000

    def bwd(q=A, k=B, v=C, out=OUT, dout=DOUT, dq=D, dk=K, dv=V, ws=WS, wb=1 << 30, d=64, tile=t):
        return lib.squad_attn_backward(p(q), p(k), p(v), p(out), p(dout), g, tile, 2, p(dq), p(dk), p(dv), 1, d, 1,
                                       ctypes.c_float(0), p(ws), wb, None)
    assert bwd(dout=0) == INVALID
    assert bwd(dv=0) == INVALID
    assert bwd(d=96) == UNSUP
    assert bwd(tile=_lib.int3((5, 4, 4))) == SHAPE
    assert bwd(dq=A) == ALIAS               # an output over an input
    assert bwd(dk=D) == ALIAS               # two outputs overlapping
    assert bwd(dv=WS) == ALIAS              # an output over the workspace
    assert bwd(ws=0) == WORKSPACE
    assert bwd(wb=need - 1) == WORKSPACE
    assert bwd(dq=D + 4) == ALIGN
    assert lib.squad_attn_forward_train(p(A), p(B), p(C), g, t, 2, p(O), 1, 64, 1, ctypes.c_float(0), p(WS),
                                        need - 1, None) == WORKSPACE
    if _device_count() == 0:
        assert bwd() == HIP


def test_block_entry_point_rejects_bad_arguments():
    lib = _lib.lib()
    p = ctypes.c_void_p
    g, t = _lib.int3((4, 8, 8)), _lib.int3((1, 4, 4))
    X, WQ, WO, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    need = sq.squad_block_workspace_size((4, 8, 8), (1, 4, 4), 2, 1, 64, 1)
    hidden = 128
    assert need >= 256 * 3 * hidden * 2 + 256 * hidden * 2   # qkv and the attention output, bf16

    # a fake, never-used rocBLAS handle: every argument check fires before the handle is touched
    def blk(x=X, wq=WQ, wo=WO, y=Y, dense=0, ws=WS, wb=1 << 30, d=64, grid=g, heads=2, blas=0x60000000):
        return lib.squad_block_forward(p(x), p(wq), p(wo), grid, t, heads, p(y), 1, d, 1, ctypes.c_float(0), dense,
                                       p(blas), p(ws), wb, None)
    assert blk(x=0) == INVALID
    assert blk(blas=0) == INVALID
    assert blk(dense=2) == INVALID
    assert blk(d=96) == UNSUP
    assert blk(y=X) == ALIAS
    assert blk(y=WQ + 64) == ALIAS
    assert blk(ws=0) == WORKSPACE
    assert blk(wb=need - 1) == WORKSPACE
    assert blk(y=Y + 8) == ALIGN
    # q, k, v rows at a stride of 3 hidden: 245,760 tokens x 3 x 3072 passes 2^31
    # elements, so the block's maps are wide; the dense comparator takes narrow maps only
    assert blk(grid=_lib.int3((64, 48, 80)), d=128, heads=24, dense=1, wb=1 << 40) == SHAPE
    assert sq.squad_block_workspace_size((64, 48, 80), (4, 12, 10), 24, 1, 128, 1) > 0
    assert sq.squad_block_workspace_size((32, 24, 40), (2, 8, 10), 24, 1, 128, 1) > 0


def test_kpass_training_argument_checks():
    lib = _lib.lib()
    p = ctypes.c_void_p
    assert sq.squad_kpass_train_workspace_size((4, 8, 8), [(1, 4, 4), (2, 2, 8)], 2, 1, 64, 1) == 0   # not nested
    need = sq.squad_kpass_train_workspace_size((4, 8, 8), [(1, 2, 2), (2, 4, 4)], 2, 1, 64, 1)
    # two fp16 intermediates, three levels of statistics, D, two gradient buffers, and
    # one inverse scale per head row of dq and of dk
    assert need == 2 * 256 * 2 * 64 * 2 + 4 * 256 * 2 * 4 + 2 * 256 * 2 * 64 * 2 + 2 * 256 * 2 * 4
    arr = (ctypes.c_int32 * 6)(1, 2, 2, 2, 4, 4)
    g = _lib.int3((4, 8, 8))
    D, K, V, OUT, DOUT = 0x60000000, 0x70000000, 0x80000000, 0x90000000, 0xA0000000

    def bwd(dq=D, ws=WS, wb=1 << 30, levels=3):
        return lib.squad_kpass_backward(p(A), p(B), p(C), p(OUT), p(DOUT), g, arr, levels, 2, p(dq), p(K), p(V), 1,
                                        64, 1, ctypes.c_float(0), p(ws), wb, None)
    assert bwd(levels=1) == INVALID
    assert bwd(dq=A) == ALIAS
    assert bwd(ws=0) == WORKSPACE
    assert bwd(wb=need - 1) == WORKSPACE
    assert lib.squad_kpass_forward_train(p(A), p(B), p(C), g, arr, 3, 2, p(O), 1, 64, 1, ctypes.c_float(0), p(WS),
                                         need - 1, None) == WORKSPACE
    if _device_count() == 0:
        assert bwd() == HIP
