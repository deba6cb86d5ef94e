"""Randomised host-side checks of the C ABI (no device needed): arbitrary, also
invalid, grids, tiles and sizes never crash the library, the workspace sizes are
zero exactly for the arguments the header rejects and otherwise the documented
byte counts, the planner's tile is valid, runs, and is no worse than simple
alternatives, and the row maps of random tilings cover each tensor's rows once.
Examples are drawn deterministically (derandomized), so a failure reproduces."""

import numpy as np
from hypothesis import HealthCheck, given, settings, strategies as st

import sub_quadratic_windowed_amd as sq

FUZZ = settings(max_examples=300, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow])


def cdiv(a, b):
    return -(-a // b)


def expected_workspace(grid, tile, heads, batch, d, dtype):
    """The forward's workspace size the header documents (0: rejected)."""
    if min(grid) <= 0 or min(tile) <= 0:
        return 0
    if heads <= 0 or batch <= 0 or d <= 0:
        return 0
    if dtype not in (0, 1) or d not in (64, 128):
        return 0
    if any(t > g for g, t in zip(grid, tile)):
        return 0
    Gp = cdiv(grid[0], tile[0]) * cdiv(grid[1], tile[1]) * cdiv(grid[2], tile[2])
    Wn = tile[0] * tile[1] * tile[2]
    cells = Gp * Wn
    if cells >= 1 << 31:
        return 0
    bh = heads * batch
    if bh * max(Gp, Wn) >= 1 << 32 or bh * cells >= 1 << 32:
        return 0
    span = cells * heads * d                      # elements per batch element
    if span >= 1 << 31 and cdiv(span, d) >= (1 << 32) - 1:
        return 0
    return bh * cells * d * (4 if dtype == 0 else 2)


axis = st.integers(min_value=-2, max_value=90)


@FUZZ
@given(grid=st.tuples(axis, axis, axis), tile=st.tuples(axis, axis, axis),
       heads=st.integers(-1, 40), batch=st.integers(-1, 3),
       d=st.sampled_from([0, 32, 64, 96, 128, 256]), dtype=st.integers(-1, 2))
def test_workspace_size_matches_the_documented_rules(grid, tile, heads, batch, d, dtype):
    got = sq.squad_attn_workspace_size(grid, tile, heads, batch, d, dtype)
    assert got == expected_workspace(grid, tile, heads, batch, d, dtype)
    train = sq.squad_attn_train_workspace_size(grid, tile, heads, batch, d, dtype)
    assert (train > 0) == (got > 0)
    if train:
        assert train >= 2 * got     # the local output and its gradient at least


def work(grid, tile):
    Gp = cdiv(grid[0], tile[0]) * cdiv(grid[1], tile[1]) * cdiv(grid[2], tile[2])
    Wn = tile[0] * tile[1] * tile[2]
    return Gp * Wn * (Gp + Wn)


@FUZZ
@given(grid=st.tuples(st.integers(1, 160), st.integers(1, 160), st.integers(1, 160)),
       probe=st.tuples(st.integers(1, 160), st.integers(1, 160), st.integers(1, 160)))
def test_planner_tile_is_valid_runs_and_beats_alternatives(grid, probe):
    tile = sq.squad_plan_tile(grid)
    assert all(1 <= t <= g for g, t in zip(grid, tile))
    assert sq.squad_attn_workspace_size(grid, tile, 24, 1, 128, 1) > 0
    w = work(grid, tile)
    alt = tuple(min(p, g) for p, g in zip(probe, grid))
    for other in (alt, grid, (1, 1, 1)):
        assert w <= work(grid, other)


small = st.integers(1, 9)


@FUZZ
@given(grid=st.tuples(small, small, small), tile=st.tuples(small, small, small),
       heads=st.integers(1, 3), batch=st.integers(1, 2), which=st.integers(0, 1))
def test_token_maps_cover_every_row_once(grid, tile, heads, batch, which):
    tile = tuple(min(t, g) for t, g in zip(tile, grid))
    d = 64
    n = grid[0] * grid[1] * grid[2]
    got = sq.squad_debug_row_offsets(which, grid, tile, heads, batch, d)
    present = got[got >= 0]
    assert np.array_equal(np.sort(present), np.arange(batch * heads * n, dtype=np.int64) * d)
    cells = 1
    for g, t in zip(grid, tile):
        cells *= cdiv(g, t) * t
    assert (got == -1).sum() == (cells - n) * heads * batch
