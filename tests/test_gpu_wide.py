"""Wide row maps on the GPU: tensors of 2^31 elements or more per batch element,
whose in-unit row offsets no longer fit 31 bits, against the float64 oracle.

64^3 tokens x 64 heads x 128 dims = 2^31 elements per tensor (4.3 GB in bf16).  Heads
are independent, so the oracle's result for the first and the last head (the last
one holds the largest offsets) is an exact reference for those heads; every element
of both is compared.  Tolerances are the other parity tests': max-abs 1.5e-2 for
bf16 forwards, 1e-4 for fp32, and for bf16 gradients 2.5e-2 of max(1, the largest
reference gradient).
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

FWD_TOL = {torch.bfloat16: 1.5e-2, torch.float32: 1e-4}
GRAD_TOL = 2.5e-2
HEADS = 64
GRID, TILE = (64, 64, 64), (4, 8, 8)       # W = 256, G = 1024
N = 64 ** 3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def randn(shape, dtype, seed):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(dtype)


def compare_heads(out, q, k, v, grid, tile, dtype, label):
    hs = [0, HEADS - 1]
    want = oracle.squad_forward(f64(q[:, :, hs]), f64(k[:, :, hs]), f64(v[:, :, hs]), grid, tile)
    got = f64(out[:, :, hs])
    err = float(np.max(np.abs(got - want)))
    say(f"  {label} heads {hs}: max-abs {err:.3e} (max |out| {np.abs(want).max():.3f})")
    assert np.isfinite(got).all()
    assert err <= FWD_TOL[dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_forward_with_wide_maps(dtype):
    shape = (1, N, HEADS, 128)
    assert N * HEADS * 128 == 1 << 31
    say(f"wide forward {dtype} {shape}")
    q, k, v = (randn(shape, dtype, 70 + i) for i in range(3))
    out = sq.squad_attn_forward(q, k, v, GRID, TILE)
    torch.cuda.synchronize()
    compare_heads(out, q, k, v, GRID, TILE, dtype, "whole")


@pytest.mark.timeout(600)
def test_forward_with_wide_maps_on_a_cut_tiling():
    """63 x 64 x 65 grid, 4 x 8 x 8 tiles: 1,296 windows of 256 cells, 262,080 tokens;
    the padded tiling's rows x 64 heads x 128 pass 2^31."""
    grid = (63, 64, 65)
    n = 63 * 64 * 65
    shape = (1, n, HEADS, 128)
    say(f"wide cut forward {shape}")
    q, k, v = (randn(shape, torch.bfloat16, 73 + i) for i in range(3))
    out = sq.squad_attn_forward(q, k, v, grid, TILE)
    torch.cuda.synchronize()
    compare_heads(out, q, k, v, grid, TILE, torch.bfloat16, "cut")


@pytest.mark.timeout(900)
def test_backward_with_wide_maps():
    shape = (1, N, HEADS, 128)
    say(f"wide backward {shape}")
    q, k, v, dout = (randn(shape, torch.bfloat16, 80 + i) for i in range(4))
    out, ws = sq.squad_attn_forward_train(q, k, v, GRID, TILE)
    dq, dk, dv = sq.squad_attn_backward(q, k, v, out, dout, GRID, TILE, ws)
    torch.cuda.synchronize()
    del ws
    hs = [0, HEADS - 1]
    qq, kk, vv, dd = (f64(x[:, :, hs]) for x in (q, k, v, dout))
    want_out = oracle.squad_forward(qq, kk, vv, GRID, TILE)
    err = float(np.max(np.abs(f64(out[:, :, hs]) - want_out)))
    say(f"  forward_train heads {hs}: max-abs {err:.3e}")
    assert err <= FWD_TOL[torch.bfloat16]
    want = oracle.squad_backward(qq, kk, vv, dd, GRID, TILE)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        g = f64(g[:, :, hs])
        e = float(np.max(np.abs(g - w)))
        ref = max(1.0, float(np.max(np.abs(w))))
        say(f"  {name}: max-abs {e:.3e} (ref max {ref:.3f})")
        assert np.isfinite(g).all()
        assert e <= GRAD_TOL * ref, (name, e)


@pytest.mark.timeout(600)
def test_permutations_with_wide_maps():
    """Gather, regroup and scatter of a 2^31-element bf16 tensor are exact: each
    equals indexing by the oracle's window partition, and the scatter undoes the
    gather."""
    shape = (1, N, HEADS, 128)
    x = randn(shape, torch.bfloat16, 90)
    idx = torch.from_numpy(oracle.window_index(GRID, TILE)).cuda()   # [G, Wn] token indices
    G, Wn = idx.shape
    say(f"wide permutations {shape}")
    win = sq.squad_tile_gather(x, GRID, TILE)                         # [B, heads, G, Wn, d]
    for h in (0, HEADS - 1):
        assert torch.equal(win[0, h], x[0, :, h][idx])
    grp = sq.squad_window_to_group(win, GRID, TILE)                   # [B, heads, Wn, G, d]
    for h in (0, HEADS - 1):
        assert torch.equal(grp[0, h], x[0, :, h][idx.t()])
    del grp
    back = sq.squad_tile_scatter(win, GRID, TILE)
    assert torch.equal(back, x)


@pytest.mark.timeout(600)
def test_block_at_the_high_resolution_shape_equals_its_parts():
    """The high-resolution block (hidden 3072 = 24 heads x 128, 64 x 48 x 80 grid, tile
    4 x 12 x 10): its q, k, v rows are read in place at a stride of 3 x 3072, so the
    in-unit offsets reach 245,760 x 9,216 > 2^31 elements and the fused path runs on
    wide maps, while the parts (contiguous q, k, v) run narrow.  The two agree to the
    bf16 rounding of their outputs."""
    grid, tile, Hh, d = (64, 48, 80), (4, 12, 10), 24, 128
    n, hidden = 245760, 3072
    gen = torch.Generator(device="cuda").manual_seed(91)
    x = torch.randn(1, n, hidden, generator=gen, device="cuda").to(torch.bfloat16)
    wqkv = (torch.randn(3 * hidden, hidden, generator=gen, device="cuda") / hidden ** 0.5).to(torch.bfloat16)
    wo = (torch.randn(hidden, hidden, generator=gen, device="cuda") / hidden ** 0.5).to(torch.bfloat16)
    say("block at the high-resolution shape")
    y = sq.squad_block_forward(x, wqkv, wo, grid, tile, Hh)
    qkv = torch.matmul(x[0], wqkv.t().contiguous())
    q, k, v = (qkv[:, i * hidden:(i + 1) * hidden].contiguous().view(1, n, Hh, d) for i in range(3))
    del qkv
    a = sq.squad_attn_forward(q, k, v, grid, tile)
    y2 = torch.matmul(a.view(n, hidden), wo.t().contiguous())
    torch.cuda.synchronize()
    diff = (y[0].float() - y2.float()).abs()
    say(f"  max |fused - parts| {float(diff.max()):.3e}, mean {float(diff.mean()):.3e}")
    assert torch.isfinite(y).all()
    assert float(diff.max()) <= 3e-2 * max(1.0, float(y2.float().abs().max()))
    assert float(diff.mean()) <= 2e-3


@pytest.mark.timeout(600)
def test_forward_with_wide_maps_head_dim_64_batch_2():
    """head_dim 64 (the row unit is then 64 elements) and two batch elements, each
    2^31 elements: 64^3 tokens x 128 heads x 64."""
    Hh = 128
    shape = (2, N, Hh, 64)
    say(f"wide forward d64 {shape}")
    q, k, v = (randn(shape, torch.bfloat16, 100 + i) for i in range(3))
    out = sq.squad_attn_forward(q, k, v, GRID, TILE)
    torch.cuda.synchronize()
    hs = [0, Hh - 1]
    want = oracle.squad_forward(f64(q[:, :, hs]), f64(k[:, :, hs]), f64(v[:, :, hs]), GRID, TILE)
    got = f64(out[:, :, hs])
    err = float(np.max(np.abs(got - want)))
    say(f"  d64 batch 2 heads {hs}: max-abs {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= FWD_TOL[torch.bfloat16]


@pytest.mark.timeout(900)
def test_backward_with_wide_maps_on_a_cut_tiling():
    grid = (63, 64, 65)
    n = 63 * 64 * 65
    shape = (1, n, HEADS, 128)
    say(f"wide cut backward {shape}")
    q, k, v, dout = (randn(shape, torch.bfloat16, 110 + i) for i in range(4))
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, TILE)
    grads = sq.squad_attn_backward(q, k, v, out, dout, grid, TILE, ws)
    torch.cuda.synchronize()
    del ws
    hs = [0, HEADS - 1]
    want = oracle.squad_backward(*(f64(x[:, :, hs]) for x in (q, k, v, dout)), grid, TILE)
    for name, g, w in zip(("dq", "dk", "dv"), grads, want):
        g = f64(g[:, :, hs])
        e = float(np.max(np.abs(g - w)))
        ref = max(1.0, float(np.max(np.abs(w))))
        say(f"  cut {name}: max-abs {e:.3e} (ref max {ref:.3f})")
        assert np.isfinite(g).all()
        assert e <= GRAD_TOL * ref, (name, e)
