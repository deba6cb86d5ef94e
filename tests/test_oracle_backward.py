"""Pins of the oracle's gradients (CPU, float64).

squad_backward is pinned to things outside itself: central finite differences of
squad_forward, torch autograd through the masked-dense statement of the operator
(tests/bruteforce.py's coordinate masks, written again in torch), and invariants
that the operator's structure fixes.  A battery of planted slips checks that the
pins catch them."""

import numpy as np
import pytest
import torch

import oracle
from oracle import squad_oracle as so
from tests import bruteforce as bf

SHAPES = [((2, 4, 6), (1, 2, 3)), ((2, 2, 3), (2, 2, 3)), ((4, 2, 2), (1, 1, 1)),   # whole tilings
          ((3, 5, 7), (2, 2, 3)), ((2, 3, 4), (2, 2, 3))]                           # cut tilings


def rand4(grid, B, Hh, d, seed, n_tensors=4):
    rng = np.random.default_rng(seed)
    n = int(np.prod(grid))
    return [rng.standard_normal((B, n, Hh, d)) for _ in range(n_tensors)]


def torch_masked_squad(q, k, v, grid, tile, scale):
    """out = A_G (A_L v) per (b, head) with A_L, A_G dense masked softmaxes in torch."""
    ml = torch.from_numpy(bf.local_mask(grid, tile))
    mg = torch.from_numpy(bf.global_mask(grid, tile))

    def attn(q, k, v, mask):
        # q, k, v: [B, n, Hh, d] -> per head dense attention
        l = scale * torch.einsum("bihd,bjhd->bhij", q, k)
        l = l.masked_fill(~mask, float("-inf"))
        a = torch.softmax(l, dim=-1)
        return torch.einsum("bhij,bjhd->bihd", a, v)

    return attn(q, k, attn(q, k, v, ml), mg)


@pytest.mark.parametrize("grid,tile", SHAPES)
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_torch_autograd_of_masked_dense(grid, tile, seed):
    q, k, v, dout = rand4(grid, 2, 2, 8, seed)
    scale = 0.41
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch_masked_squad(tq, tk, tv, grid, tile, scale)
    out.backward(torch.from_numpy(dout))
    dq, dk, dv = oracle.squad_backward(q, k, v, dout, grid, tile, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("grid,tile", [SHAPES[0], SHAPES[3]])
def test_backward_matches_central_differences(grid, tile):
    """Directional derivatives of <dout, squad_forward> along random directions."""
    q, k, v, dout = rand4(grid, 1, 2, 4, 5)
    grads = oracle.squad_backward(q, k, v, dout, grid, tile)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for which in range(3):
        for _ in range(3):
            u = rng.standard_normal(q.shape)
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = args_p[which] + eps * u
            args_m[which] = args_m[which] - eps * u
            fd = (np.sum(dout * oracle.squad_forward(*args_p, grid, tile))
                  - np.sum(dout * oracle.squad_forward(*args_m, grid, tile))) / (2 * eps)
            assert abs(fd - np.sum(grads[which] * u)) <= 1e-7 * max(1.0, abs(fd))


def test_backward_elementwise_central_differences_tiny():
    grid, tile = (1, 2, 4), (1, 2, 2)
    q, k, v, dout = rand4(grid, 1, 1, 2, 6)
    grads = oracle.squad_backward(q, k, v, dout, grid, tile)
    eps = 1e-6
    for which in range(3):
        x = [q, k, v][which]
        for idx in np.ndindex(x.shape):
            e = np.zeros_like(x)
            e[idx] = eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which] = x + e
            args_m[which] = x - e
            fd = (np.sum(dout * oracle.squad_forward(*args_p, grid, tile))
                  - np.sum(dout * oracle.squad_forward(*args_m, grid, tile))) / (2 * eps)
            assert abs(fd - grads[which][idx]) <= 1e-8


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_backward_invariants(grid, tile):
    q, k, v, dout = rand4(grid, 2, 3, 8, 2)
    dq, dk, dv = oracle.squad_backward(q, k, v, dout, grid, tile)
    # out = M v with M row-stochastic: the value gradient keeps the column sums
    np.testing.assert_allclose(dv.sum(axis=1), dout.sum(axis=1), atol=1e-11)
    # adding one vector to every key shifts each logit row by a constant: no effect
    np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)
    # constant values: the output is that constant whatever q and k are
    vc = np.broadcast_to(v[:, :1], v.shape).copy()
    dq0, dk0, _ = oracle.squad_backward(q, k, vc, dout, grid, tile)
    np.testing.assert_allclose(dq0, 0.0, atol=1e-11)
    np.testing.assert_allclose(dk0, 0.0, atol=1e-11)
    # zero queries: logits do not depend on k
    _, dkz, _ = oracle.squad_backward(np.zeros_like(q), k, v, dout, grid, tile)
    np.testing.assert_allclose(dkz, 0.0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_pass_backwards_match_torch_autograd(grid, tile):
    """Each pass's gradient alone (the value stream of the global pass is free)."""
    q, k, v, dout = rand4(grid, 1, 2, 8, 3)
    s = 0.3
    for fn, mask, bwd in ((oracle.local_pass, bf.local_mask, oracle.local_pass_backward),
                          (oracle.global_pass, bf.global_mask, oracle.global_pass_backward)):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        m = torch.from_numpy(mask(grid, tile))
        l = (s * torch.einsum("bihd,bjhd->bhij", tq, tk)).masked_fill(~m, float("-inf"))
        out = torch.einsum("bhij,bjhd->bihd", torch.softmax(l, -1), tv)
        np.testing.assert_allclose(fn(q, k, v, grid, tile, s), out.detach().numpy(), atol=1e-12)
        out.backward(torch.from_numpy(dout))
        for got, want in zip(bwd(q, k, v, dout, grid, tile, s), (tq.grad, tk.grad, tv.grad)):
            np.testing.assert_allclose(got, want.numpy(), atol=1e-12)


@pytest.mark.parametrize("grid,tile", SHAPES)
def test_forward_stats_are_masked_logsumexp(grid, tile):
    q, k, _, _ = rand4(grid, 1, 2, 8, 4)
    s = 0.5
    lse_l, lse_g = oracle.squad_forward_stats(q, k, grid, tile, s)
    for lse, mask in ((lse_l, bf.local_mask(grid, tile)), (lse_g, bf.global_mask(grid, tile))):
        for h in range(2):
            l = s * q[0, :, h] @ k[0, :, h].T
            want = np.log(np.where(mask, np.exp(l), 0.0).sum(axis=1))
            np.testing.assert_allclose(lse[0, :, h], want, atol=1e-12)


# ---------------------------------------------------------------- planted slips

def backward_battery():
    for grid, tile in (SHAPES[0], SHAPES[3]):
        q, k, v, dout = rand4(grid, 1, 2, 8, 7)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        torch_masked_squad(tq, tk, tv, grid, tile, 0.35).backward(torch.from_numpy(dout))
        for got, want in zip(so.squad_backward(q, k, v, dout, grid, tile, 0.35), (tq.grad, tk.grad, tv.grad)):
            np.testing.assert_allclose(got, want.numpy(), atol=1e-10)


def _no_centering(q, k, v, dout, scale):
    q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
    l = float(scale) * q @ np.swapaxes(k, -1, -2)
    a = np.exp(l - l.max(-1, keepdims=True))
    a /= a.sum(-1, keepdims=True)
    dl = a * (dout @ np.swapaxes(v, -1, -2))
    return float(scale) * dl @ k, float(scale) * np.swapaxes(dl, -1, -2) @ q, np.swapaxes(a, -1, -2) @ dout


BACKWARD_MUTANTS = {
    "softmax Jacobian without the row term": lambda mp: mp.setattr(so, "softmax_attention_backward", _no_centering),
    "dq and dk swapped": lambda mp: mp.setattr(
        so, "softmax_attention_backward",
        (lambda f: (lambda *a: (lambda r: (r[1], r[0], r[2]))(f(*a))))(so.softmax_attention_backward)),
    "scale missing from dk": lambda mp: mp.setattr(
        so, "softmax_attention_backward",
        (lambda f: (lambda q, k, v, d, s: (lambda r: (r[0], r[1] / s, r[2]))(f(q, k, v, d, s))))(
            so.softmax_attention_backward)),
    "global pass's q gradient dropped": lambda mp: mp.setattr(
        so, "global_pass_backward",
        (lambda f: (lambda *a, **kw: (lambda r: (0 * r[0], r[1], r[2]))(f(*a, **kw))))(so.global_pass_backward)),
    "local pass fed dout instead of the local output's gradient": lambda mp: mp.setattr(
        so, "squad_backward",
        lambda q, k, v, dout, g, t, s=None: tuple(
            a + b for a, b in zip(so.global_pass_backward(q, k, so.local_pass(q, k, v, g, t, s), dout, g, t, s)[:2],
                                  so.local_pass_backward(q, k, v, dout, g, t, s)[:2]))
        + (so.local_pass_backward(q, k, v, dout, g, t, s)[2],)),
}


def test_backward_battery_passes_on_the_real_oracle():
    backward_battery()


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTANTS))
def test_backward_battery_rejects_mutant(name, monkeypatch):
    BACKWARD_MUTANTS[name](monkeypatch)
    with pytest.raises(AssertionError):
        backward_battery()
