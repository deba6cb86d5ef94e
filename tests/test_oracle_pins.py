"""Pins of the float64 oracle against facts fixed by the pages and by mathematics.

Each test would fail under a plausible slip in the oracle: a dropped scale, a
softmax over the wrong axis, a wrong index map, the global pass grouped by window
instead of by offset, the value stream taken from v instead of the local output,
or the token order transposed.  None of these tests re-types the oracle's formula.
"""

import glob
import json
import os

import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# (grid, tile) pairs: cubic and non-cubic tiles, degenerate G = 1 and W = 1 cases
SHAPES = [
    ((4, 8, 8), (1, 4, 4)),
    ((2, 2, 2), (1, 1, 2)),
    ((2, 4, 6), (2, 2, 3)),
    ((3, 2, 4), (1, 2, 2)),
    ((1, 4, 4), (1, 4, 4)),   # G = 1: one window
    ((2, 3, 4), (1, 1, 1)),   # W = 1: one token per window
    ((4, 3, 5), (2, 1, 5)),
    ((6, 2, 2), (3, 2, 1)),
]


def rand_qkv(shape, B, Hh, d, seed, dist="normal"):
    g = np.random.default_rng(seed)
    n = int(np.prod(shape))
    q = g.standard_normal((B, n, Hh, d))
    k = g.standard_normal((B, n, Hh, d))
    v = g.standard_normal((B, n, Hh, d))
    if dist == "peaky":
        q *= g.uniform(0.5, 2.0, (B, n, Hh, 1)) * 2.0
        k *= g.uniform(0.5, 2.0, (B, n, Hh, 1)) * 2.0
    return q, k, v


def sdpa64(q, k, v, scale):
    """torch's own scaled-dot-product attention in float64 on the CPU: [B,n,Hh,d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float64).transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


# ---------------------------------------------------------------- golden (hand-derived)

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "closed_form_*.json"))))
def test_golden_closed_forms(path):
    fx = json.load(open(path))
    q = np.array(fx["q"], np.float64)[None, :, None, :]
    k = np.array(fx["k"], np.float64)[None, :, None, :]
    v = np.array(fx["v"], np.float64)[None, :, None, :]
    out = oracle.squad_forward(q, k, v, fx["grid"], fx["tile"], fx["scale"])
    np.testing.assert_allclose(out[0, :, 0, :], np.array(fx["out"]), rtol=0, atol=1e-12)
    if "o1" in fx:
        o1 = oracle.local_pass(q, k, v, fx["grid"], fx["tile"], fx["scale"])
        np.testing.assert_allclose(o1[0, :, 0, :], np.array(fx["o1"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- index map

@pytest.mark.parametrize("grid,tile", SHAPES)
def test_window_index_is_the_tile_partition(grid, tile):
    idx = oracle.window_index(grid, tile)
    n = int(np.prod(grid))
    G, Wn = idx.shape
    assert G * Wn == n and Wn == int(np.prod(tile))
    assert np.array_equal(np.sort(idx.ravel()), np.arange(n))          # a permutation
    # every window is one tile: all its members share the coordinate-derived window id
    wid, off = bf.window_id(grid, tile), bf.offset_id(grid, tile)
    assert all(len(set(wid[idx[g]])) == 1 for g in range(G))
    assert np.array_equal(wid[idx[:, 0]], np.arange(G))
    # column p holds exactly the tokens with offset p, one per window
    assert all(np.all(off[idx[:, p]] == p) for p in range(Wn))


def test_window_index_rejects_ragged_grid():
    with pytest.raises(ValueError):
        oracle.window_index((4, 8, 8), (3, 4, 4))


# ---------------------------------------------------------------- brute force (masked dense)

@pytest.mark.parametrize("grid,tile", SHAPES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_oracle_matches_masked_dense_bruteforce(grid, tile, seed):
    B, Hh, d = 2, 2, 8
    q, k, v = rand_qkv(grid, B, Hh, d, seed, "peaky" if seed == 2 else "normal")
    s = 0.37
    out = oracle.squad_forward(q, k, v, grid, tile, s)
    ref, ref_o1 = bf.squad_bruteforce(q, k, v, grid, tile, s)
    np.testing.assert_allclose(oracle.local_pass(q, k, v, grid, tile, s), ref_o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES[:4])
def test_stages_match_masked_dense_separately(grid, tile):
    """Global pass alone, fed an arbitrary value stream, equals the strided-mask attention."""
    q, k, v = rand_qkv(grid, 1, 3, 4, 7)
    s = 0.5
    AL, AG = bf.matrices(q, k, grid, tile, s)
    g = oracle.global_pass(q, k, v, grid, tile, s)
    for h in range(3):
        np.testing.assert_allclose(g[0, :, h], AG[0, h] @ v[0, :, h], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- degenerate tiles reduce to full attention

@pytest.mark.parametrize("grid", [(4, 8, 8), (2, 3, 5), (1, 1, 7)])
def test_single_window_is_full_attention(grid):
    """tile = grid: the local pass is full attention, the global pass is a softmax over one token."""
    q, k, v = rand_qkv(grid, 2, 2, 16, 3)
    out = oracle.squad_forward(q, k, v, grid, grid)
    np.testing.assert_allclose(out, sdpa64(q, k, v, 1 / 4), rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid", [(4, 8, 8), (2, 3, 5)])
def test_single_token_windows_is_full_attention(grid):
    """tile = 1x1x1: the local pass is the identity, the global pass is full attention."""
    q, k, v = rand_qkv(grid, 1, 3, 16, 4)
    out = oracle.squad_forward(q, k, v, grid, (1, 1, 1))
    np.testing.assert_allclose(oracle.local_pass(q, k, v, grid, (1, 1, 1)), v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out, sdpa64(q, k, v, 1 / 4), rtol=0, atol=1e-12)


def test_dense_attention_is_sdpa():
    q, k, v = rand_qkv((2, 4, 4), 2, 3, 32, 5)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v), sdpa64(q, k, v, 32 ** -0.5), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v, 0.1), sdpa64(q, k, v, 0.1), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants and closed forms

@pytest.mark.parametrize("grid,tile", SHAPES)
def test_constant_values_give_constant_output(grid, tile):
    q, k, _ = rand_qkv(grid, 1, 2, 8, 11, "peaky")
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25, 3.0, 0, 1, 2, 3]), q.shape).copy()
    out = oracle.squad_forward(q, k, v, grid, tile)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_zero_queries_give_window_mean_then_global_mean(grid, tile):
    """q = 0: every logit is 0, so the local output is the window mean of v and
    the output is the mean of v over all n tokens (groups all have G members and
    every window contributes one member)."""
    _, k, v = rand_qkv(grid, 2, 2, 8, 12)
    q = np.zeros_like(k)
    idx = oracle.window_index(grid, tile)
    o1 = oracle.local_pass(q, k, v, grid, tile)
    for g in range(idx.shape[0]):
        np.testing.assert_allclose(o1[:, idx[g]], np.broadcast_to(v[:, idx[g]].mean(1, keepdims=True), o1[:, idx[g]].shape), atol=1e-12)
    out = oracle.squad_forward(q, k, v, grid, tile)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(1, keepdims=True), out.shape), rtol=0, atol=1e-12)


def test_linear_in_values():
    grid, tile = (2, 4, 6), (2, 2, 3)
    q, k, v1 = rand_qkv(grid, 1, 2, 8, 13)
    _, _, v2 = rand_qkv(grid, 1, 2, 8, 14)
    f = lambda v: oracle.squad_forward(q, k, v, grid, tile)
    np.testing.assert_allclose(f(2.5 * v1 - 0.75 * v2), 2.5 * f(v1) - 0.75 * f(v2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", [((2, 2, 4), (1, 2, 2)), ((2, 3, 2), (2, 1, 2)), ((1, 4, 4), (1, 2, 2))])
def test_effective_matrix_full_receptive_field(grid, tile):
    """v = identity: out is the effective mixing matrix E = A_G A_L.  Every token
    reaches every other (full receptive field), rows sum to 1, and each pair (i, j)
    is joined by exactly one path, through k* = the member of j's window that
    shares i's offset."""
    n = int(np.prod(grid))
    g = np.random.default_rng(15)
    q = g.standard_normal((1, n, 1, 4))
    k = g.standard_normal((1, n, 1, 4))
    v = np.eye(n)[None, :, None, :]                      # head_dim = n
    s = 0.5
    E = oracle.squad_forward(np.pad(q, ((0, 0), (0, 0), (0, 0), (0, n - 4))),
                             np.pad(k, ((0, 0), (0, 0), (0, 0), (0, n - 4))), v, grid, tile, s)[0, :, 0, :]
    assert np.all(E > 0)
    np.testing.assert_allclose(E.sum(1), 1.0, atol=1e-12)
    AL, AG = bf.matrices(q, k, grid, tile, s)
    wid, off = bf.window_id(grid, tile), bf.offset_id(grid, tile)
    for i in range(n):
        for j in range(n):
            kstar = np.flatnonzero((wid == wid[j]) & (off == off[i]))
            assert kstar.size == 1
            assert np.isclose(E[i, j], AG[0, 0, i, kstar[0]] * AL[0, 0, kstar[0], j], rtol=1e-12, atol=0)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_equivariant_under_flips_and_tile_rolls(axis):
    grid, tile = (4, 6, 6), (2, 3, 2)
    q, k, v = rand_qkv(grid, 1, 2, 8, 16)
    f = lambda x: oracle.squad_forward(*x, grid, tile)
    to5 = lambda x: x.reshape(1, *grid, 2, 8)
    fr5 = lambda x: x.reshape(1, -1, 2, 8)
    out = to5(f((q, k, v)))
    flip = lambda x: fr5(np.flip(to5(x), axis=1 + axis))
    np.testing.assert_allclose(to5(f(tuple(flip(x) for x in (q, k, v)))), np.flip(out, axis=1 + axis), atol=1e-12)
    roll = lambda x: fr5(np.roll(to5(x), tile[axis], axis=1 + axis))
    np.testing.assert_allclose(to5(f(tuple(roll(x) for x in (q, k, v)))), np.roll(out, tile[axis], axis=1 + axis), atol=1e-12)


def test_not_equivariant_under_sub_tile_roll():
    """A roll by less than a tile changes the partition, so the output is not a roll
    of the original output: the operator really depends on the window layout."""
    grid, tile = (2, 4, 4), (1, 2, 2)
    q, k, v = rand_qkv(grid, 1, 1, 8, 17)
    to5 = lambda x: x.reshape(1, *grid, 1, 8)
    roll = lambda x: np.roll(to5(x), 1, axis=3).reshape(1, -1, 1, 8)
    out = oracle.squad_forward(q, k, v, grid, tile)
    out_r = oracle.squad_forward(roll(q), roll(k), roll(v), grid, tile)
    assert not np.allclose(out_r, roll(out), atol=1e-6)


def test_large_logits_stay_finite():
    grid, tile = (2, 4, 4), (1, 2, 2)
    q, k, v = rand_qkv(grid, 1, 2, 8, 18)
    out = oracle.squad_forward(q, k, v, grid, tile, 300.0)
    assert np.all(np.isfinite(out))
    ref, _ = bf.squad_bruteforce(q, k, v, grid, tile, 300.0)
    np.testing.assert_allclose(out, ref, atol=1e-10)


# ---------------------------------------------------------------- sampled groups, reshapes

@pytest.mark.parametrize("grid,tile", SHAPES)
def test_groups_equal_full_forward_rows(grid, tile):
    q, k, v = rand_qkv(grid, 2, 2, 8, 19)
    out = oracle.squad_forward(q, k, v, grid, tile)
    Wn = int(np.prod(tile))
    ps = sorted({0, Wn - 1, Wn // 2})
    tokens, rows = oracle.squad_forward_groups(q, k, v, grid, tile, ps)
    for i in range(len(ps)):
        np.testing.assert_allclose(rows[:, i], out[:, tokens[i]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_reshapes_are_the_coordinate_permutation(grid, tile):
    B, Hh, d = 2, 3, 4
    x = np.arange(B * int(np.prod(grid)) * Hh * d).reshape(B, -1, Hh, d)
    y = oracle.tile_gather(x, grid, tile)
    wid, off = bf.window_id(grid, tile), bf.offset_id(grid, tile)
    for i in range(x.shape[1]):
        assert np.array_equal(y[:, :, wid[i], off[i]], x[:, i])
    assert np.array_equal(oracle.tile_scatter(y, grid, tile), x)
    z = oracle.window_to_group(y)
    assert np.array_equal(z[:, :, off, wid], x.transpose(0, 2, 1, 3))


def test_window_attn_rows_are_convex_combinations():
    g = np.random.default_rng(20)
    q, k, v = (g.standard_normal((5, 7, 16)) for _ in range(3))
    o = oracle.window_attn(q, k, v)
    assert np.all(o <= v.max(1, keepdims=True) + 1e-12) and np.all(o >= v.min(1, keepdims=True) - 1e-12)
    np.testing.assert_allclose(o, sdpa64(q[:, :, None], k[:, :, None], v[:, :, None], 0.25)[:, :, 0], atol=1e-12)


# ---------------------------------------------------------------- tilings cut by the grid edge

# (grid, tile) pairs whose grid is not a whole number of tiles: cuts along one, two
# and three axes, a tile as large as the grid along an axis, single-token edge windows
CUT_SHAPES = [
    ((3, 5, 7), (2, 2, 3)),
    ((4, 6, 5), (3, 4, 2)),
    ((5, 5, 5), (2, 3, 4)),
    ((2, 4, 7), (2, 4, 3)),   # cut along w only
    ((3, 3, 3), (2, 2, 2)),   # the corner window holds one token
    ((1, 5, 6), (1, 5, 4)),
]


@pytest.mark.parametrize("grid,tile", CUT_SHAPES)
def test_padded_window_index_is_the_cut_partition(grid, tile):
    idx = oracle.padded_window_index(grid, tile)
    n = int(np.prod(grid))
    present = idx[idx >= 0]
    assert np.array_equal(np.sort(present), np.arange(n))              # every token once
    wid, off = bf.window_id(grid, tile), bf.offset_id(grid, tile)
    G, Wn = idx.shape
    assert Wn == int(np.prod(tile))
    for g in range(G):
        row = idx[g][idx[g] >= 0]
        assert row.size > 0 and np.all(wid[row] == g)
        # a window holds the tile's box clipped by the grid: the product of the clipped extents
        t0 = (g // (-(-grid[1] // tile[1]) * -(-grid[2] // tile[2]))) * tile[0]
        h0 = (g // -(-grid[2] // tile[2])) % -(-grid[1] // tile[1]) * tile[1]
        w0 = g % -(-grid[2] // tile[2]) * tile[2]
        ext = [min(tile[0], grid[0] - t0), min(tile[1], grid[1] - h0), min(tile[2], grid[2] - w0)]
        assert row.size == int(np.prod(ext))
    for p in range(Wn):
        col = idx[:, p][idx[:, p] >= 0]
        assert np.all(off[col] == p)


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_padded_window_index_on_whole_tilings(grid, tile):
    assert np.array_equal(oracle.padded_window_index(grid, tile), oracle.window_index(grid, tile))


@pytest.mark.parametrize("grid,tile", CUT_SHAPES)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cut_tiling_matches_masked_dense_bruteforce(grid, tile, seed):
    B, Hh, d = 2, 2, 8
    q, k, v = rand_qkv(grid, B, Hh, d, seed, "peaky" if seed == 2 else "normal")
    s = 0.41
    ref, ref_o1 = bf.squad_bruteforce(q, k, v, grid, tile, s)
    np.testing.assert_allclose(oracle.local_pass(q, k, v, grid, tile, s), ref_o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.squad_forward(q, k, v, grid, tile, s), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES[:4])
def test_per_unit_path_equals_batched_path_on_whole_tilings(grid, tile):
    """The per-unit path that serves cut tilings, run on a whole tiling, gives the
    batched path's result (the same operator, computed unit by unit)."""
    q, k, v = rand_qkv(grid, 1, 2, 8, 5)
    idx = oracle.padded_window_index(grid, tile)
    s = 0.5
    np.testing.assert_allclose(oracle.squad_oracle._unit_attention(q, k, v, idx, s),
                               oracle.local_pass(q, k, v, grid, tile, s), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.squad_oracle._unit_attention(q, k, v, idx.T, s),
                               oracle.global_pass(q, k, v, grid, tile, s), rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", CUT_SHAPES)
def test_cut_tiling_zero_queries_closed_form(grid, tile):
    """q = 0: the local output is the mean of v over the token's (clipped) window,
    and the output is the plain mean, over the windows present in the token's
    offset group, of those window means; computed here from coordinates."""
    q, _, v = rand_qkv(grid, 1, 1, 4, 7)
    q = np.zeros_like(q)
    k = np.random.default_rng(8).standard_normal(q.shape)
    out = oracle.squad_forward(q, k, v, grid, tile, 0.9)
    wid, off = bf.window_id(grid, tile), bf.offset_id(grid, tile)
    wmean = {g: v[0, wid == g, 0].mean(axis=0) for g in np.unique(wid)}
    for i in range(int(np.prod(grid))):
        members = np.flatnonzero(off == off[i])                # the group of token i
        expect = np.mean([wmean[wid[j]] for j in members], axis=0)
        np.testing.assert_allclose(out[0, i, 0], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", CUT_SHAPES[:3])
def test_cut_tiling_constant_values(grid, tile):
    q, k, _ = rand_qkv(grid, 1, 2, 4, 3)
    v = np.full_like(q, -1.25)
    np.testing.assert_allclose(oracle.squad_forward(q, k, v, grid, tile), v, rtol=0, atol=1e-12)
