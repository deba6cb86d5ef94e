"""Pins of the oracle's k-pass operator (CPU, float64): k = 2 is the two-pass
operator; masked dense brute force with one coordinate mask per level; a level
of size one drops out; partitions, closed forms and planted slips."""

import numpy as np
import pytest

import oracle
from oracle import squad_oracle as so
from tests import bruteforce as bf

KCASES = [((4, 8, 8), [(1, 2, 2), (2, 4, 4)]),           # k = 3
          ((2, 6, 6), [(1, 1, 1), (1, 3, 3)]),           # level 0 of size one
          ((4, 4, 8), [(1, 2, 2), (2, 2, 4), (2, 4, 8)]),  # k = 4
          ((3, 4, 6), [(1, 2, 3)]),                       # k = 2
          ((2, 8, 4), [(2, 2, 1), (2, 4, 2)])]


def rand_qkv(grid, B, Hh, d, seed):
    rng = np.random.default_rng(seed)
    n = int(np.prod(grid))
    return [rng.standard_normal((B, n, Hh, d)) for _ in range(3)]


def level_digits(grid, tiles):
    """Per-token digit of every level on every axis, from coordinates."""
    t, h, w = bf.coords(grid)
    ext = [(1, 1, 1)] + [tuple(x) for x in tiles] + [tuple(grid)]
    out = []
    for j in range(len(ext) - 1):
        out.append(np.stack([(c // ext[j][a]) % (ext[j + 1][a] // ext[j][a]) for a, c in enumerate((t, h, w))], -1))
    return out


def kpass_bruteforce(q, k, v, grid, tiles, scale):
    """Dense n x n softmax per pass; pass j's mask: all digits but level j's equal."""
    dig = level_digits(grid, tiles)
    o = np.asarray(v, np.float64)
    B, n, Hh, d = o.shape
    for j in range(len(dig)):
        mask = np.ones((n, n), bool)
        for l, dl in enumerate(dig):
            if l != j:
                mask &= (dl[:, None, :] == dl[None, :, :]).all(-1)
        nxt = np.empty_like(o)
        for b in range(B):
            for h in range(Hh):
                a = bf.masked_attention_matrix(q[b, :, h], k[b, :, h], mask, scale)
                nxt[b, :, h] = a @ o[b, :, h]
        o = nxt
    return o


@pytest.mark.parametrize("grid,tiles", KCASES)
def test_kpass_matches_masked_dense_bruteforce(grid, tiles):
    q, k, v = rand_qkv(grid, 2, 2, 8, 0)
    np.testing.assert_allclose(oracle.squad_kpass_forward(q, k, v, grid, tiles, 0.4),
                               kpass_bruteforce(q, k, v, grid, tiles, 0.4), atol=1e-12)


@pytest.mark.parametrize("grid,tile", [((4, 8, 8), (1, 4, 4)), ((2, 4, 6), (2, 2, 3)), ((3, 6, 4), (3, 2, 4))])
def test_two_levels_are_the_two_pass_operator(grid, tile):
    q, k, v = rand_qkv(grid, 1, 3, 16, 1)
    np.testing.assert_allclose(oracle.squad_kpass_forward(q, k, v, grid, [tile]),
                               oracle.squad_forward(q, k, v, grid, tile), atol=1e-13)


def test_a_level_of_size_one_drops_out():
    grid = (4, 8, 8)
    q, k, v = rand_qkv(grid, 1, 2, 8, 2)
    three = oracle.squad_kpass_forward(q, k, v, grid, [(1, 4, 4), (1, 4, 4)])
    two = oracle.squad_kpass_forward(q, k, v, grid, [(1, 4, 4)])
    np.testing.assert_allclose(three, two, atol=1e-13)
    first = oracle.squad_kpass_forward(q, k, v, grid, [(1, 1, 1), (1, 4, 4)])
    np.testing.assert_allclose(first, two, atol=1e-13)


@pytest.mark.parametrize("grid,tiles", KCASES)
def test_levels_partition_the_tokens(grid, tiles):
    n = int(np.prod(grid))
    for level in range(len(tiles) + 1):
        idx = oracle.kpass_level_index(grid, tiles, level)
        assert np.array_equal(np.sort(idx.ravel()), np.arange(n))
    # two tokens share a unit in every level but the ones where their digits differ:
    # over all levels, a pair of distinct tokens shares exactly k - (#differing levels) units
    dig = level_digits(grid, tiles)
    i, j = 0, n - 1
    differ = sum(not np.array_equal(d[i], d[j]) for d in dig)
    shared = sum(any(i in row and j in row for row in oracle.kpass_level_index(grid, tiles, l))
                 for l in range(len(dig)))
    assert shared == (1 if differ == 1 else 0)


@pytest.mark.parametrize("grid,tiles", KCASES[:3])
def test_kpass_closed_forms(grid, tiles):
    q, k, v = rand_qkv(grid, 1, 2, 8, 3)
    # constant values stay constant
    vc = np.broadcast_to(v[:, :1], v.shape).copy()
    np.testing.assert_allclose(oracle.squad_kpass_forward(q, k, vc, grid, tiles), vc, atol=1e-12)
    # zero queries: every pass averages uniformly, so the result is the mean of v over all tokens
    out = oracle.squad_kpass_forward(np.zeros_like(q), k, v, grid, tiles)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(axis=1, keepdims=True), v.shape), atol=1e-12)


def test_composed_passes_reach_every_token():
    """The effective matrix of the composition is strictly positive: every output
    token depends on every input token (full receptive field at any depth)."""
    grid, tiles = (2, 4, 4), [(1, 2, 2), (2, 2, 4)]
    q, k, _ = rand_qkv(grid, 1, 1, 4, 4)
    n = 32
    eye = np.eye(n)[None, :, None, :]           # v = identity columns (d = n)
    qq = np.concatenate([q] * (n // 4), axis=-1)
    kk = np.concatenate([k] * (n // 4), axis=-1)
    m = oracle.squad_kpass_forward(qq, kk, eye, grid, tiles, 0.3)[0, :, 0, :]
    assert (m > 0).all()
    np.testing.assert_allclose(m.sum(axis=1), 1.0, atol=1e-12)


def test_rejects_tiles_that_do_not_nest():
    q, k, v = rand_qkv((4, 8, 8), 1, 1, 4, 5)
    with pytest.raises(ValueError):
        oracle.squad_kpass_forward(q, k, v, (4, 8, 8), [(1, 4, 4), (2, 2, 8)])


# ---------------------------------------------------------------- planted slips

def kpass_battery():
    for grid, tiles in KCASES[:3]:
        q, k, v = rand_qkv(grid, 1, 2, 8, 6)
        np.testing.assert_allclose(so.squad_kpass_forward(q, k, v, grid, tiles, 0.4),
                                   kpass_bruteforce(q, k, v, grid, tiles, 0.4), atol=1e-10)


KMUTANTS = {
    "passes in reverse order": lambda mp: mp.setattr(
        so, "kpass_level_index",
        (lambda f: (lambda g, t, l: f(g, t, len(t) - l)))(so.kpass_level_index)),
    "last pass skipped": lambda mp: mp.setattr(
        so, "squad_kpass_forward",
        (lambda f: (lambda q, k, v, g, t, s=None: f(q, k, v, g, t[:-1], s)))(so.squad_kpass_forward)),
    "middle pass grouped like the first": lambda mp: mp.setattr(
        so, "kpass_level_index",
        (lambda f: (lambda g, t, l: f(g, t, 0 if l == 1 and len(t) > 1 else l)))(so.kpass_level_index)),
}


def test_kpass_battery_passes_on_the_real_oracle():
    kpass_battery()


@pytest.mark.parametrize("name", sorted(KMUTANTS))
def test_kpass_battery_rejects_mutant(name, monkeypatch):
    KMUTANTS[name](monkeypatch)
    with pytest.raises((AssertionError, ValueError)):
        kpass_battery()


# ---------------------------------------------------------------- the attention block (oracle)

def test_block_with_identity_projections_is_the_operator():
    grid, tile, heads, d = (2, 4, 6), (2, 2, 3), 2, 4
    hidden = heads * d
    rng = np.random.default_rng(7)
    x = rng.standard_normal((1, 48, hidden))
    eye = np.eye(hidden)
    y = oracle.squad_block_forward(x, np.concatenate([eye, eye, eye]), eye, grid, tile, heads)
    xh = x.reshape(1, 48, heads, d)
    np.testing.assert_allclose(y, oracle.squad_forward(xh, xh, xh, grid, tile).reshape(1, 48, hidden), atol=1e-13)


def test_block_projections_enter_as_plain_products():
    """Zero query weights: every pass averages uniformly, so y is the mean over all
    tokens of x w_v^T, through w_out (a closed form of the three products)."""
    grid, tile, heads, d = (2, 4, 6), (2, 2, 3), 2, 4
    hidden = heads * d
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 48, hidden))
    wq = np.zeros((hidden, hidden))
    wk, wv, wo = (rng.standard_normal((hidden, hidden)) for _ in range(3))
    y = oracle.squad_block_forward(x, np.concatenate([wq, wk, wv]), wo, grid, tile, heads)
    want = (x @ wv.T).mean(axis=1, keepdims=True) @ wo.T
    np.testing.assert_allclose(y, np.broadcast_to(want, y.shape), atol=1e-12)
    # dense comparator with a single window equals the operator (tile = grid)
    w = np.concatenate([rng.standard_normal((hidden, hidden)) for _ in range(3)])
    np.testing.assert_allclose(oracle.squad_block_forward(x, w, wo, grid, grid, heads),
                               oracle.squad_block_forward(x, w, wo, grid, tile, heads, dense=True), atol=1e-12)


# ---------------------------------------------------------------- k-pass gradients (oracle)

def torch_kpass(q, k, v, grid, tiles, scale):
    """The k-pass operator as dense masked attentions in torch (one mask per level)."""
    import torch
    dig = level_digits(grid, tiles)
    n = q.shape[1]
    o = v
    for j in range(len(dig)):
        mask = np.ones((n, n), bool)
        for l, dl in enumerate(dig):
            if l != j:
                mask &= (dl[:, None, :] == dl[None, :, :]).all(-1)
        m = torch.from_numpy(mask)
        lg = (scale * torch.einsum("bihd,bjhd->bhij", q, k)).masked_fill(~m, float("-inf"))
        o = torch.einsum("bhij,bjhd->bihd", torch.softmax(lg, -1), o)
    return o


@pytest.mark.parametrize("grid,tiles", KCASES)
def test_kpass_backward_matches_torch_autograd(grid, tiles):
    import torch
    q, k, v = rand_qkv(grid, 2, 2, 8, 11)
    dout = np.random.default_rng(12).standard_normal(q.shape)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    torch_kpass(tq, tk, tv, grid, tiles, 0.45).backward(torch.from_numpy(dout))
    got = oracle.squad_kpass_backward(q, k, v, dout, grid, tiles, 0.45)
    for g, w in zip(got, (tq.grad, tk.grad, tv.grad)):
        np.testing.assert_allclose(g, w.numpy(), atol=1e-12)


def test_kpass_backward_two_levels_is_the_two_pass_backward():
    grid, tile = (4, 8, 8), (1, 4, 4)
    q, k, v = rand_qkv(grid, 1, 2, 8, 13)
    dout = np.random.default_rng(14).standard_normal(q.shape)
    for a, b in zip(oracle.squad_kpass_backward(q, k, v, dout, grid, [tile]),
                    oracle.squad_backward(q, k, v, dout, grid, tile)):
        np.testing.assert_allclose(a, b, atol=1e-13)


def test_kpass_backward_central_differences():
    grid, tiles = (2, 4, 4), [(1, 2, 2), (2, 2, 4)]
    q, k, v = rand_qkv(grid, 1, 1, 4, 15)
    dout = np.random.default_rng(16).standard_normal(q.shape)
    grads = oracle.squad_kpass_backward(q, k, v, dout, grid, tiles)
    rng = np.random.default_rng(17)
    eps = 1e-6
    for which in range(3):
        u = rng.standard_normal(q.shape)
        p_ = [q, k, v]
        m_ = [q, k, v]
        p_[which] = p_[which] + eps * u
        m_[which] = m_[which] - eps * u
        fd = (np.sum(dout * oracle.squad_kpass_forward(*p_, grid, tiles))
              - np.sum(dout * oracle.squad_kpass_forward(*m_, grid, tiles))) / (2 * eps)
        assert abs(fd - np.sum(grads[which] * u)) <= 1e-7 * max(1.0, abs(fd))
