"""Full-size parity: every output element of the three large workloads, and every
gradient element at the high-resolution unit sizes, against the float64 oracle.

The oracle runs over a few heads at a time (heads are independent), so its
memory stays bounded while every (token, head) output is compared.  Tolerances
are the ones of the other parity tests: max-abs 1.5e-2 for bf16 forwards, and for
gradients 2.5e-2 of max(1, the largest reference gradient).
"""

import sys
import time

import numpy as np
import pytest
import torch

import oracle
from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

FWD_TOL = 1.5e-2
GRAD_TOL = 2.5e-2


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


def check_grads(got, want, label):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        g = f64(g)
        err = float(np.max(np.abs(g - w)))
        ref = max(1.0, float(np.max(np.abs(w))))
        rms = float(np.sqrt(np.mean((g - w) ** 2)) / max(1e-30, np.sqrt(np.mean(w ** 2))))
        say(f"  {label} {name}: max-abs {err:.3e} (ref max {ref:.3f}), rel-rms {rms:.3e}")
        assert np.isfinite(g).all(), name
        assert err <= GRAD_TOL * ref, (name, err)


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["dit5b_bf16", "long_bf16", "highres_bf16"])
def test_every_output_element_at_full_size(name):
    """The configuration's own seeded inputs (24 heads), the forward in the bench's
    launch configuration, and the oracle's forward four heads at a time: every one
    of the B * n * heads * head_dim outputs is compared."""
    cfg = inputs.CONFIGS[name]
    say(f"{name}: generating inputs {cfg.shape}")
    qc, kc, vc = inputs.config_inputs(cfg)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    out = sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads)
    torch.cuda.synchronize()
    outc = out.cpu()
    del q, k, v, out
    torch.cuda.empty_cache()
    worst, compared = 0.0, 0
    step = 4
    for h0 in range(0, cfg.heads, step):
        hs = slice(h0, min(h0 + step, cfg.heads))
        t0 = time.time()
        want = oracle.squad_forward(f64(qc[:, :, hs]), f64(kc[:, :, hs]), f64(vc[:, :, hs]), cfg.grid, cfg.tile)
        err = float(np.max(np.abs(f64(outc[:, :, hs]) - want)))
        worst = max(worst, err)
        compared += want.size
        say(f"  heads {hs.start}-{hs.stop - 1}: max-abs {err:.3e} (max |out| {np.abs(want).max():.3f}), "
            f"oracle {time.time() - t0:.1f} s")
    say(f"  {name}: {compared} outputs, max-abs {worst:.3e}")
    assert compared == cfg.batch * cfg.n * cfg.heads * cfg.head_dim
    assert worst <= FWD_TOL


@pytest.mark.timeout(1200)
def test_backward_at_the_high_resolution_unit_sizes():
    """The high-resolution grid and tile (64x48x80, 4x12x10: local units of 480 rows,
    global units of 512, exactly the backward's row-table size) with 2 heads; every
    element of dq, dk, dv against the oracle's gradients."""
    cfg = inputs.CONFIGS["highres_bf16"]
    shape = (1, cfg.n, 2, 128)
    q, k, v = (x.cuda() for x in inputs.make_qkv(shape, torch.bfloat16, False, 38))
    g = torch.Generator().manual_seed(1038)
    dout = torch.randn(shape, generator=g).to(torch.bfloat16).cuda()
    say("backward at the high-resolution unit sizes, 2 heads")
    out, ws = sq.squad_attn_forward_train(q, k, v, cfg.grid, cfg.tile)
    grads = sq.squad_attn_backward(q, k, v, out, dout, cfg.grid, cfg.tile, ws)
    torch.cuda.synchronize()
    t0 = time.time()
    want = oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), cfg.grid, cfg.tile)
    say(f"  oracle {time.time() - t0:.1f} s")
    check_grads(grads, want, "highres units")


@pytest.mark.timeout(600)
def test_backward_with_row_offsets_past_2_to_the_30():
    """32,768 tokens x 384 heads x 128 dims = 1.61e9 elements per tensor: the global
    pass's in-unit row offsets reach 1.41e9 elements (past 2^30), so their byte
    offsets need all 32 unsigned bits.  Heads are independent, so the oracle's
    gradients of the first and the last head are exact references for those
    heads; every element of both is compared, forward output included."""
    grid, tile, Hh, d = (32, 32, 32), (4, 8, 8), 384, 128
    n = 32 * 32 * 32
    gen = torch.Generator(device="cuda").manual_seed(62)
    q, k, v, dout = (torch.randn(1, n, Hh, d, generator=gen, device="cuda").to(torch.bfloat16) for _ in range(4))
    say("backward with row offsets past 2^30: forward_train + backward")
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    dq, dk, dv = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws)
    torch.cuda.synchronize()
    del ws
    hs = [0, Hh - 1]
    qq, kk, vv, dd = (f64(x[:, :, hs]) for x in (q, k, v, dout))
    want_out = oracle.squad_forward(qq, kk, vv, grid, tile)
    err = float(np.max(np.abs(f64(out[:, :, hs]) - want_out)))
    say(f"  forward heads {hs}: max-abs {err:.3e}")
    assert err <= FWD_TOL
    want = oracle.squad_backward(qq, kk, vv, dd, grid, tile)
    check_grads((dq[:, :, hs], dk[:, :, hs], dv[:, :, hs]), want, f"heads {hs}")
    del q, k, v, dout, out, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_the_planners_tile_for_65_cubed():
    """65 x 65 x 65 = 274,625 tokens has no whole tiling near sqrt(n); the planner
    picks 3 x 13 x 13, a cut tiling of 550 windows of 507 cells (both passes past
    the 512-row tables).  Forward and gradients, 2 heads, every element against the
    oracle."""
    grid = (65, 65, 65)
    tile = sq.squad_plan_tile(grid)
    assert tile == (3, 13, 13)
    n = 65 ** 3
    shape = (1, n, 2, 128)
    q, k, v = (x.cuda() for x in inputs.make_qkv(shape, torch.bfloat16, True, 63))
    g = torch.Generator().manual_seed(1063)
    dout = torch.randn(shape, generator=g).to(torch.bfloat16).cuda()
    say(f"planner tile for {grid}: {tile}")
    out = sq.squad_attn_forward(q, k, v, grid, tile)
    out_t, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    grads = sq.squad_attn_backward(q, k, v, out_t, dout, grid, tile, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)
    qq, kk, vv, dd = f64(q), f64(k), f64(v), f64(dout)
    t0 = time.time()
    want = oracle.squad_forward(qq, kk, vv, grid, tile)
    err = float(np.max(np.abs(f64(out) - want)))
    say(f"  forward max-abs {err:.3e} (oracle {time.time() - t0:.1f} s)")
    assert np.isfinite(f64(out)).all() and err <= FWD_TOL
    check_grads(grads, oracle.squad_backward(qq, kk, vv, dd, grid, tile), "65^3")


def test_local_output_near_the_top_of_fp16():
    """The local output is held in fp16 between the passes, so values must stay
    below 65504 in magnitude (the documented precondition).  v drawn in [-3.99, 3.99]
    and scaled by 2^14 (exact in bf16) reaches 65,372: outputs and gradients stay
    finite, and the errors scale with v (the bf16 tolerance times 2^14 for the
    output; the gradient bound is already relative to the largest gradient)."""
    grid, tile, Hh, d = (4, 6, 10), (2, 3, 5), 2, 128
    n = 240
    q, k, v = inputs.make_qkv((1, n, Hh, d), torch.bfloat16, True, 39)
    v = (v.float().clamp(-3.99, 3.99) * 2.0 ** 14).to(torch.bfloat16)
    assert float(v.float().abs().max()) < 65504
    g = torch.Generator().manual_seed(1039)
    dout = torch.randn((1, n, Hh, d), generator=g).to(torch.bfloat16)
    q, k, v, dout = (x.cuda() for x in (q, k, v, dout))
    out = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
    out_t, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    grads = sq.squad_attn_backward(q, k, v, out_t, dout, grid, tile, ws)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    got = f64(out)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - want)))
    say(f"  |v| up to {float(v.float().abs().max()):.0f}: forward max-abs {err:.3e} "
        f"(bound {FWD_TOL * 2 ** 14:.1f}, max |out| {np.abs(want).max():.0f})")
    assert err <= FWD_TOL * 2.0 ** 14
    assert torch.equal(out, out_t)
    check_grads(grads, oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), grid, tile), "fp16 range")
