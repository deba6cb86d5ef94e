"""Seeded random shapes against the float64 oracle: grids of 1-24 cells per axis,
tiles anywhere from one cell to the whole grid (whole and cut tilings), batch 1-2,
1-3 heads, head_dim 64 or 128, fp32 and bf16.  Forward on 24 shapes, forward_train
plus backward on 12; the tolerances are the other parity tests'."""

import sys

import numpy as np
import pytest
import torch

import oracle
from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

FWD_TOL = {torch.float32: 1e-4, torch.bfloat16: 1.5e-2}
GRAD_TOL = {torch.float32: 1e-4, torch.bfloat16: 2.5e-2}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def random_cases(seed, count, max_tokens):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        grid = tuple(int(x) for x in rng.integers(1, 25, size=3))
        n = grid[0] * grid[1] * grid[2]
        if n > max_tokens:
            continue
        if rng.random() < 0.5:   # a whole tiling: each tile extent divides the grid's
            tile = tuple(int(rng.choice([t for t in range(1, g + 1) if g % t == 0])) for g in grid)
        else:
            tile = tuple(int(rng.integers(1, g + 1)) for g in grid)
        dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
        cases.append((grid, tile, int(rng.integers(1, 3)), int(rng.integers(1, 4)),
                      int(rng.choice([64, 128])), dtype, bool(rng.random() < 0.5)))
    return cases


def case_id(c):
    return f"{c[0]}-{c[1]}-b{c[2]}h{c[3]}d{c[4]}-{str(c[5])[6:]}{'-peaky' if c[6] else ''}"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


@pytest.mark.parametrize("case", random_cases(2024, 24, 6000), ids=case_id)
def test_random_shape_forward(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = (x.cuda() for x in inputs.make_qkv((B, n, Hh, d), dtype, peaky, 160))
    out = sq.squad_attn_forward(q, k, v, grid, tile)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    got = f64(out)
    err = float(np.max(np.abs(got - want)))
    say(f"  {case_id(case)}: max-abs {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= FWD_TOL[dtype]


@pytest.mark.parametrize("case", random_cases(2025, 12, 3000), ids=case_id)
def test_random_shape_backward(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    shape = (B, n, Hh, d)
    q, k, v = (x.cuda() for x in inputs.make_qkv(shape, dtype, peaky, 161))
    dout = torch.randn(shape, generator=torch.Generator().manual_seed(162)).to(dtype).cuda()
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    grads = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws)
    torch.cuda.synchronize()
    want = oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), grid, tile)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        g = f64(g)
        err = float(np.max(np.abs(g - w)))
        ref = max(1.0, float(np.max(np.abs(w))))
        say(f"  {case_id(case)} {name}: max-abs {err:.3e} (ref max {ref:.3f})")
        assert np.isfinite(g).all()
        assert err <= GRAD_TOL[dtype] * ref, (name, err)
