"""GPU parity of the k-pass operator (squad_kpass_forward) against the float64
oracle, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

import oracle
from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.bfloat16: 1.5e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def rand_inputs(shape, dtype, seed, peaky=False):
    return tuple(x.cuda() for x in inputs.make_qkv(shape, dtype, peaky, seed))


KCASES = [
    # grid, tiles, batch, heads, head_dim, dtype, peaky
    ((4, 8, 8), [(1, 2, 2), (2, 4, 4)], 1, 2, 64, torch.float32, False),          # k = 3, units of 4, 8, 8
    ((4, 8, 8), [(1, 2, 2), (2, 4, 4)], 2, 3, 128, torch.bfloat16, True),
    ((4, 4, 8), [(1, 2, 2), (2, 2, 4), (2, 4, 8)], 1, 2, 128, torch.bfloat16, False),  # k = 4
    ((8, 16, 20), [(2, 4, 5), (4, 8, 10)], 1, 2, 128, torch.bfloat16, False),     # units 40, 8, 8
    ((8, 12, 20), [(2, 3, 4), (4, 6, 20)], 1, 2, 64, torch.bfloat16, True),       # units 24, 20, 4
    ((16, 16, 16), [(4, 4, 4), (8, 8, 8)], 1, 1, 128, torch.bfloat16, False),     # units 64, 8, 8
    ((2, 24, 40), [(1, 8, 10), (2, 24, 40)], 1, 1, 128, torch.bfloat16, False),   # last level of size one
    ((4, 6, 10), [(1, 3, 5), (2, 6, 10)], 1, 2, 128, torch.float32, False),       # units 15, 8, 2
    ((2, 32, 32), [(1, 1, 1), (2, 32, 32)], 1, 2, 128, torch.bfloat16, False),    # middle level of 2048 rows
]


@pytest.mark.parametrize("case", KCASES, ids=lambda c: f"{c[0]}-k{len(c[1]) + 1}-d{c[4]}-{str(c[5])[6:]}")
def test_kpass_matches_oracle(case):
    grid, tiles, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 41, peaky)
    say(f"kpass {case}")
    out = sq.squad_kpass_forward(q, k, v, grid, tiles)
    torch.cuda.synchronize()
    want = oracle.squad_kpass_forward(f64(q), f64(k), f64(v), grid, tiles)
    err = float(np.max(np.abs(f64(out) - want)))
    say(f"  max-abs {err:.3e}")
    assert np.isfinite(f64(out)).all()
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_two_levels_are_the_forward_bit_for_bit(dtype):
    grid, tile = (8, 12, 10), (2, 6, 5)
    q, k, v = rand_inputs((2, 960, 3, 128), dtype, 42, True)
    a = sq.squad_kpass_forward(q, k, v, grid, [tile])
    b = sq.squad_attn_forward(q, k, v, grid, tile)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_a_repeated_tile_is_a_pass_of_size_one():
    """A level whose tile equals the next one has units of one row: that pass copies
    its value stream exactly, so the result equals the operator without it."""
    grid = (4, 8, 8)
    q, k, v = rand_inputs((1, 256, 2, 128), torch.bfloat16, 43)
    a = sq.squad_kpass_forward(q, k, v, grid, [(1, 2, 2), (1, 2, 2), (2, 4, 4)])
    b = sq.squad_kpass_forward(q, k, v, grid, [(1, 2, 2), (2, 4, 4)])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_kpass_at_highres_size_properties():
    """Three levels over the high-resolution grid (units of 64, 64 and 60 tokens, 4
    heads): constant values stay constant and q = 0 gives the mean of v, to the
    fp16 / bf16 rounding of the intermediate and final outputs."""
    cfg = inputs.CONFIGS["highres_bf16"]
    tiles = [(4, 4, 4), (16, 16, 16)]
    q, k, v = rand_inputs((1, cfg.n, 4, 128), torch.bfloat16, 44)
    say("kpass highres properties")
    vc = v[:, :1].expand_as(v).contiguous()
    outc = sq.squad_kpass_forward(q, k, vc, cfg.grid, tiles)
    outz = sq.squad_kpass_forward(torch.zeros_like(q), k, v, cfg.grid, tiles)
    torch.cuda.synchronize()
    assert float((outc.float() - vc.float()).abs().max()) <= 1.5e-2
    mean = v.double().mean(dim=1, keepdim=True)
    assert float((outz.double() - mean).abs().max()) <= 1.5e-2


# ---------------------------------------------------------------- k-level training

KBWD_CASES = [
    ((4, 8, 8), [(1, 2, 2), (2, 4, 4)], 1, 2, 64, torch.float32),
    ((4, 8, 8), [(1, 2, 2), (2, 4, 4)], 2, 2, 128, torch.bfloat16),
    ((4, 4, 8), [(1, 2, 2), (2, 2, 4), (2, 4, 8)], 1, 2, 128, torch.bfloat16),   # two middle levels
    ((8, 16, 20), [(2, 4, 5), (4, 8, 10)], 1, 2, 128, torch.bfloat16),
    ((4, 6, 10), [(1, 3, 5), (2, 6, 10)], 1, 2, 64, torch.float32),
]


@pytest.mark.parametrize("case", KBWD_CASES, ids=lambda c: f"{c[0]}-k{len(c[1]) + 1}-d{c[4]}-{str(c[5])[6:]}")
def test_kpass_backward_matches_oracle(case):
    grid, tiles, B, Hh, d, dtype = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 45)
    g = torch.Generator().manual_seed(46)
    dout = torch.randn(B, n, Hh, d, generator=g).to(dtype).cuda()
    say(f"kpass backward {case}")
    out, ws = sq.squad_kpass_forward_train(q, k, v, grid, tiles)
    grads = sq.squad_kpass_backward(q, k, v, out, dout, grid, tiles, ws)
    ref = sq.squad_kpass_forward(q, k, v, grid, tiles)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    want = oracle.squad_kpass_backward(f64(q), f64(k), f64(v), f64(dout), grid, tiles)
    tol = 1e-4 if dtype == torch.float32 else 2.5e-2
    for name, got, w in zip(("dq", "dk", "dv"), grads, want):
        err = float(np.max(np.abs(f64(got) - w)))
        bound = tol * max(1.0, float(np.max(np.abs(w))))
        say(f"  {name}: max-abs {err:.3e} (bound {bound:.3e})")
        assert np.isfinite(f64(got)).all() and err <= bound


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_kpass_backward_two_levels_is_the_two_pass_backward(dtype):
    """Two levels run the same kernels as squad_attn_backward with the local output
    in token order instead of group-major: the same bits."""
    grid, tile = (4, 6, 10), (2, 3, 5)
    q, k, v = rand_inputs((2, 240, 2, 128), dtype, 47)
    dout = torch.randn(2, 240, 2, 128, generator=torch.Generator().manual_seed(48)).to(dtype).cuda()
    out, ws = sq.squad_kpass_forward_train(q, k, v, grid, [tile])
    a = sq.squad_kpass_backward(q, k, v, out, dout, grid, [tile], ws)
    out2, ws2 = sq.squad_attn_forward_train(q, k, v, grid, tile)
    b = sq.squad_attn_backward(q, k, v, out2, dout, grid, tile, ws2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
