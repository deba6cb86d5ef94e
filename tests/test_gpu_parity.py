"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerances are max-abs: 1e-4 for fp32 inputs, 1.5e-2 for bf16 inputs with fp32
accumulation.  The oracle is always fed the exact values the GPU saw (bf16 inputs
upcast exactly).  Integer and byte work (the permutations) must be bit-exact.
"""

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


def dev(x):
    return x.cuda()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def maxerr(got, want):
    return float(np.max(np.abs(f64(got) - want))) if np.size(want) else 0.0


def rand_inputs(shape, dtype, seed, peaky=False):
    return tuple(dev(x) for x in inputs.make_qkv(shape, dtype, peaky, seed))


# ---------------------------------------------------------------- full forward, small shapes vs full oracle

FORWARD_CASES = [
    # grid, tile, batch, heads, head_dim, dtype, peaky
    ((4, 8, 8), (1, 4, 4), 1, 2, 64, torch.float32, False),      # the tiny fp32 configuration's shape
    ((4, 8, 8), (1, 4, 4), 2, 3, 128, torch.float32, True),
    ((4, 6, 10), (2, 3, 5), 1, 3, 128, torch.float32, False),    # W = 30, G = 8: ragged key blocks
    ((4, 6, 10), (2, 3, 5), 2, 3, 128, torch.bfloat16, True),
    ((8, 8, 8), (2, 4, 4), 1, 2, 64, torch.bfloat16, False),     # W = 32, G = 16
    ((6, 10, 10), (2, 5, 10), 1, 2, 128, torch.bfloat16, False), # W = 100, G = 6
    ((8, 12, 10), (1, 12, 10), 1, 2, 128, torch.bfloat16, True), # W = 120, G = 8
    ((2, 16, 20), (2, 8, 10), 1, 2, 128, torch.bfloat16, False), # W = 160, G = 4
    ((16, 8, 8), (1, 1, 1), 1, 2, 128, torch.bfloat16, False),   # W = 1, G = 1024
    ((4, 8, 8), (4, 8, 8), 1, 2, 64, torch.bfloat16, False),     # G = 1: one window
    ((3, 5, 7), (3, 5, 7), 1, 1, 64, torch.float32, False),      # G = 1, n = 105
    ((4, 16, 20), (4, 8, 10), 1, 1, 128, torch.bfloat16, True),  # W = 320 (5 chunks of key blocks)
    ((8, 24, 20), (2, 12, 10), 1, 1, 128, torch.bfloat16, False),# W = 240, G = 16
]


@pytest.mark.parametrize("case", FORWARD_CASES, ids=lambda c: f"{c[0]}-{c[1]}-b{c[2]}h{c[3]}d{c[4]}-{str(c[5])[6:]}")
def test_forward_matches_oracle(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 7, peaky)
    say(f"forward {case}")
    out = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    err = maxerr(out, want)
    say(f"  max-abs {err:.3e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("scale", [0.3, 1e-3], ids=["scale0.3", "scale1e-3"])
def test_forward_custom_scale(dtype, scale):
    """A caller-given softmax scale reaches both passes (1e-3 makes both passes
    nearly uniform averages)."""
    grid, tile = (4, 6, 10), (2, 3, 5)
    q, k, v = rand_inputs((1, 240, 2, 128), dtype, 11)
    out = sq.squad_attn_forward(q, k, v, grid, tile, 2, scale=scale)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile, scale=scale)
    assert maxerr(out, want) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_forward_window_beyond_row_tables(dtype):
    """W = 576 rows per window: the local pass locates rows without the per-unit
    LDS tables (more than 512 rows), the global pass has G = 2 rows per group."""
    grid, tile = (4, 12, 24), (4, 12, 12)
    q, k, v = rand_inputs((1, 1152, 2, 128), dtype, 12)
    out = sq.squad_attn_forward(q, k, v, grid, tile, 2)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    assert maxerr(out, want) <= TOL[dtype]


def test_forward_sharp_attention_rescales():
    """q and k scaled by 4: logits with a standard deviation near 16, so the running
    maximum is raised (and the accumulator rescaled) in the middle of units."""
    grid, tile = (4, 16, 20), (4, 8, 10)
    q, k, v = rand_inputs((1, 1280, 2, 128), torch.bfloat16, 13)
    q, k = q * 4, k * 4   # exact in bf16 (a power of two)
    out = sq.squad_attn_forward(q, k, v, grid, tile, 2)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    assert np.isfinite(f64(out)).all()
    assert maxerr(out, want) <= TOL[torch.bfloat16]


def test_forward_reuses_buffers():
    """Two calls with the same preallocated output and workspace, the second on other
    inputs, each match the oracle (nothing from the first call leaks into the second)."""
    grid, tile = (4, 6, 10), (2, 3, 5)
    shape = (1, 240, 3, 128)
    ws = torch.empty(sq.squad_attn_workspace_size(grid, tile, 3, 1, 128, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for seed in (14, 15):
        q, k, v = rand_inputs(shape, torch.bfloat16, seed, peaky=True)
        sq.squad_attn_forward(q, k, v, grid, tile, 3, out=out, workspace=ws)
        torch.cuda.synchronize()
        want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
        assert maxerr(out, want) <= TOL[torch.bfloat16]


@pytest.mark.parametrize("case", FORWARD_CASES[:8], ids=lambda c: f"{c[0]}-{c[1]}-{str(c[5])[6:]}")
def test_each_pass_matches_oracle(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 8, peaky)
    o1 = sq.squad_local_pass(q, k, v, grid, tile, Hh)
    out = sq.squad_global_pass(q, k, v, grid, tile, Hh)   # arbitrary value stream: v itself
    torch.cuda.synchronize()
    qq, kk, vv = f64(q), f64(k), f64(v)
    assert maxerr(o1, oracle.local_pass(qq, kk, vv, grid, tile)) <= TOL[dtype]
    assert maxerr(out, oracle.global_pass(qq, kk, vv, grid, tile)) <= TOL[dtype]


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16"])
def test_config_forward_matches_oracle(name):
    cfg = inputs.CONFIGS[name]
    q, k, v = (dev(x) for x in inputs.config_inputs(cfg))
    say(f"config {name}")
    out = sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), cfg.grid, cfg.tile)
    err = maxerr(out, want)
    say(f"  max-abs {err:.3e} (max |out| {np.abs(want).max():.3f})")
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("seed", range(1, 10))
def test_config_seed_sweep(seed):
    """The tiny and small configurations over more seeds."""
    for name in ("tiny_fp32", "small_bf16"):
        cfg = inputs.CONFIGS[name]
        q, k, v = (dev(x) for x in inputs.config_inputs(cfg, seed=seed))
        out = sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads)
        torch.cuda.synchronize()
        if name == "small_bf16":   # the full oracle at 24 heads costs a few seconds; check 4 heads
            hs = [0, 7, 13, 23]
            want = oracle.squad_forward(f64(q[:, :, hs]), f64(k[:, :, hs]), f64(v[:, :, hs]), cfg.grid, cfg.tile)
            err = maxerr(out[:, :, hs], want)
        else:
            err = maxerr(out, oracle.squad_forward(f64(q), f64(k), f64(v), cfg.grid, cfg.tile))
        assert err <= TOL[cfg.dtype], (name, seed, err)


# ---------------------------------------------------------------- full-size configurations, sampled

@pytest.mark.parametrize("name", ["dit5b_bf16", "long_bf16", "highres_bf16"])
def test_large_config_sampled_groups(name):
    """At full size the oracle computes whole offset groups (every token of the group,
    each through its own window) for a sample of groups and heads."""
    cfg = inputs.CONFIGS[name]
    say(f"config {name}: generating inputs")
    qc, kc, vc = inputs.config_inputs(cfg)
    q, k, v = dev(qc), dev(kc), dev(vc)
    say("  running the forward")
    out = sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads)
    torch.cuda.synchronize()
    W = cfg.window
    offsets = [0, 1, W // 2, W - 1]
    hs = [0, cfg.heads // 2, cfg.heads - 1]
    say("  oracle on sampled groups")
    tokens, want = oracle.squad_forward_groups(qc[:, :, hs].double().numpy(), kc[:, :, hs].double().numpy(),
                                               vc[:, :, hs].double().numpy(), cfg.grid, cfg.tile, offsets)
    got = out[:, torch.from_numpy(tokens.reshape(-1)).cuda()][:, :, hs]
    got = got.reshape(cfg.batch, len(offsets), -1, len(hs), cfg.head_dim)
    err = maxerr(got, want)
    say(f"  max-abs {err:.3e} over {want.size} outputs")
    assert err <= TOL[cfg.dtype]
    del q, k, v, out
    torch.cuda.empty_cache()


def test_largest_row_offsets_sampled_groups():
    """Rows addressed with 32-bit in-unit offsets close to their limit: 262,144 tokens
    x 48 heads x 128 dims = 1.61e9 elements per tensor (the host rejects 2^31), and
    G = 1024 offsets per group, past the global pass's LDS row tables.  The oracle
    checks whole offset groups of the first and the last head (the largest
    offsets) on a sample of offsets."""
    grid, tile, Hh, d = (64, 64, 64), (4, 8, 8), 48, 128
    n = 64 * 64 * 64
    g = torch.Generator(device="cuda").manual_seed(61)
    q, k, v = (torch.randn(1, n, Hh, d, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    say("largest offsets: running the forward")
    out = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
    torch.cuda.synchronize()
    offsets = [0, 255]
    for h in (0, Hh - 1):
        say(f"  oracle on head {h}")
        tokens, want = oracle.squad_forward_groups(f64(q[:, :, h:h + 1]), f64(k[:, :, h:h + 1]),
                                                   f64(v[:, :, h:h + 1]), grid, tile, offsets)
        got = out[:, torch.from_numpy(tokens.reshape(-1)).cuda(), h:h + 1]
        got = got.reshape(1, len(offsets), -1, 1, d)
        err = maxerr(got, want)
        scale = float(np.max(np.abs(want)))
        say(f"  head {h}: max-abs {err:.3e} over {want.size} outputs (max |out| {scale:.3f})")
        assert err <= TOL[torch.bfloat16]
        # outputs here average hundreds of values (max |out| ~ 0.2), so also hold the
        # error to a few bf16 ulps of the output scale: a misplaced row would be off
        # by the order of that scale
        assert err <= 2e-2 * scale
    del q, k, v, out
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- properties at full size (no oracle)

def test_highres_properties():
    cfg = inputs.CONFIGS["highres_bf16"]
    qc, kc, vc = inputs.config_inputs(cfg)
    q, k, v = dev(qc), dev(kc), dev(vc)
    g, t = cfg.grid, cfg.tile
    ws = torch.empty(sq.squad_attn_workspace_size(g, t, cfg.heads, 1, 128, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = sq.squad_attn_forward(q, k, v, g, t, workspace=ws)
    # determinism: a second run is bit-identical
    out2 = sq.squad_attn_forward(q, k, v, g, t, workspace=ws)
    assert torch.equal(out, out2)
    # linear in v: doubling v doubles the output (exactly, except where the fp16 local
    # output is subnormal, below 6.1e-5, and doubling it is not exact)
    out3 = sq.squad_attn_forward(q, k, v * 2, g, t, workspace=ws)
    two = 2 * out.float()
    assert float(((out3.float() - two).abs() - two.abs() * 2.0 ** -7).max()) <= 1e-6   # within one bf16 ulp
    assert float((out3 == 2 * out).float().mean()) > 0.99
    del out2, out3
    # constant values give that constant back
    ones = torch.full_like(v, 1.0)
    oc = sq.squad_attn_forward(q, k, ones, g, t, workspace=ws)
    assert float((oc.float() - 1).abs().max()) <= TOL[torch.bfloat16]
    del oc, ones
    # q = 0: the output is the mean of v over all tokens, per head
    oz = sq.squad_attn_forward(torch.zeros_like(q), k, v, g, t, workspace=ws)
    mean = v.float().mean(dim=1, keepdim=True)
    assert float((oz.float() - mean).abs().max()) <= TOL[torch.bfloat16]
    del oz
    # a roll of the grid by one tile along each axis rolls the output the same way
    shp = (1, *g, cfg.heads, 128)
    for ax in range(3):
        sh = t[ax]
        roll = lambda x: torch.roll(x.reshape(shp), sh, dims=1 + ax).reshape(x.shape).contiguous()
        orl = sq.squad_attn_forward(roll(q), roll(k), roll(v), g, t, workspace=ws)
        assert float((orl.float() - roll(out).float()).abs().max()) <= TOL[torch.bfloat16]
        del orl


# ---------------------------------------------------------------- the engine and the comparator

# L spans every shape of the block loop: 1-2 blocks (2-wave workgroups), 3-5 blocks (no
# round with all successors), 6-9 blocks (one such round, then the last round and a
# remainder of 0-2 blocks), 15-16 blocks (the full-size units) and beyond the row tables
@pytest.mark.parametrize("L", [1, 17, 64, 65, 96, 100, 160, 192, 200, 256, 288, 384, 480, 512, 600])
@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_window_attn_matches_oracle(L, dtype, d):
    U = 40
    g = torch.Generator().manual_seed(L)
    q, k, v = (torch.randn(U, L, d, generator=g).to(dtype).cuda() for _ in range(3))
    o = sq.squad_window_attn(q, k, v)
    torch.cuda.synchronize()
    assert maxerr(o, oracle.window_attn(f64(q), f64(k), f64(v))) <= TOL[dtype]


@pytest.mark.parametrize("n,dtype", [(1024, torch.bfloat16), (1000, torch.bfloat16), (333, torch.float32)])
def test_dense_matches_oracle(n, dtype):
    q, k, v = rand_inputs((2, n, 3, 128), dtype, 9)
    o = sq.squad_dense_attn_forward(q, k, v)
    torch.cuda.synchronize()
    assert maxerr(o, oracle.dense_attention(f64(q), f64(k), f64(v))) <= TOL[dtype]


def test_single_window_equals_dense_kernel():
    """tile = grid: SQuad reduces to full attention; compare with the dense kernel."""
    grid = (4, 16, 16)
    q, k, v = rand_inputs((1, 1024, 2, 128), torch.bfloat16, 10)
    a = sq.squad_attn_forward(q, k, v, grid, grid)
    b = sq.squad_dense_attn_forward(q, k, v)
    torch.cuda.synchronize()
    assert float((a.float() - b.float()).abs().max()) <= TOL[torch.bfloat16]


# ---------------------------------------------------------------- permutations: bit-exact

PERM_CASES = [((4, 8, 8), (1, 4, 4), 2, 3, 64, torch.bfloat16), ((2, 4, 6), (2, 2, 3), 1, 2, 128, torch.float32),
              ((32, 24, 40), (2, 8, 10), 1, 24, 128, torch.bfloat16), ((4, 6, 10), (1, 1, 1), 1, 2, 64, torch.float32),
              ((4, 6, 10), (4, 6, 10), 1, 2, 128, torch.bfloat16)]


@pytest.mark.parametrize("case", PERM_CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def test_permutations_are_exact(case):
    grid, tile, B, Hh, d, dtype = case
    n = grid[0] * grid[1] * grid[2]
    x = torch.randn(B, n, Hh, d).to(dtype)
    xg = x.cuda()
    w = sq.squad_tile_gather(xg, grid, tile)
    want_w = oracle.tile_gather(x.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), grid, tile)
    as_int = lambda t: t.cpu().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(as_int(w), want_w)
    back = sq.squad_tile_scatter(w, grid, tile)
    assert torch.equal(back, xg)
    grp = sq.squad_window_to_group(w, grid, tile)
    assert np.array_equal(as_int(grp), oracle.window_to_group(want_w))


def test_forward_halves_compose_to_the_forward():
    """squad_attn_forward == squad_attn_forward_local then squad_attn_forward_global, bit for bit."""
    grid, tile = (8, 12, 10), (2, 6, 5)
    q, k, v = rand_inputs((2, 960, 3, 128), torch.bfloat16, 11, True)
    out = sq.squad_attn_forward(q, k, v, grid, tile)
    ws = sq.squad_attn_forward_local(q, k, v, grid, tile)
    out2 = sq.squad_attn_forward_global(q, k, grid, tile, ws)
    assert torch.equal(out, out2)
    # the workspace holds the local output, group-major [B, heads, Wn, G, d], in fp16
    o1 = ws.view(torch.float16).reshape(2, 3, 60, 16, 128)
    want = oracle.tile_gather(oracle.local_pass(f64(q), f64(k), f64(v), grid, tile), grid, tile)
    assert maxerr(o1.transpose(2, 3), want) <= TOL[torch.bfloat16]


# ---------------------------------------------------------------- cut tilings (grid not a whole number of tiles)

CUT_CASES = [
    # grid, tile, batch, heads, head_dim, dtype, peaky
    ((3, 5, 7), (2, 2, 3), 1, 2, 64, torch.float32, False),       # cut on every axis, Wn = 12, G = 18
    ((3, 5, 7), (2, 2, 3), 2, 2, 128, torch.bfloat16, True),
    ((5, 12, 20), (2, 5, 6), 1, 2, 128, torch.bfloat16, False),   # Wn = 60, G = 36
    ((5, 12, 20), (2, 5, 6), 1, 1, 64, torch.float32, True),
    ((4, 8, 8), (3, 4, 4), 1, 2, 64, torch.bfloat16, False),      # cut along t only
    ((7, 7, 7), (1, 2, 7), 1, 2, 128, torch.bfloat16, False),     # the planner's tile for 7^3
    ((9, 19, 21), (5, 10, 10), 1, 2, 128, torch.bfloat16, False), # Wn = 500 (16 key blocks), G = 12
    ((3, 17, 30), (2, 16, 16), 1, 1, 64, torch.bfloat16, True),   # Wn = 512, G = 8
    ((8, 15, 15), (1, 2, 2), 1, 2, 128, torch.bfloat16, False),   # G = 512 groups of 1..4 present rows
    ((9, 32, 32), (2, 1, 1), 1, 1, 64, torch.float32, False),     # fp32: G = 5120 rows per group
    ((21, 45, 79), (3, 9, 10), 1, 2, 128, torch.bfloat16, False), # n = 74655, Wn = 270, G = 280, cut along w
    ((5, 13, 20), (4, 12, 12), 1, 2, 128, torch.bfloat16, True),  # Wn = 576: local units past the row tables
    ((9, 31, 40), (2, 2, 2), 1, 2, 128, torch.bfloat16, False),   # G = 1600: global units past the row tables
]


@pytest.mark.parametrize("case", CUT_CASES, ids=lambda c: f"{c[0]}-{c[1]}-b{c[2]}h{c[3]}d{c[4]}-{str(c[5])[6:]}")
def test_cut_forward_matches_oracle(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 21, peaky)
    say(f"cut forward {case}")
    out = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
    torch.cuda.synchronize()
    want = oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)
    err = maxerr(out, want)
    say(f"  max-abs {err:.3e}")
    assert np.isfinite(f64(out)).all()
    assert err <= TOL[dtype]


@pytest.mark.parametrize("case", CUT_CASES[:6], ids=lambda c: f"{c[0]}-{c[1]}-{str(c[5])[6:]}")
def test_cut_each_pass_matches_oracle(case):
    """The half-pass entry points on cut tilings, every present token written."""
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((B, n, Hh, d), dtype, 22, peaky)
    say(f"cut passes {case}")
    nanfill = torch.full((B, n, Hh, d), float("nan"), dtype=dtype, device="cuda")
    o1 = sq.squad_local_pass(q, k, v, grid, tile, Hh, out=nanfill.clone())
    out = sq.squad_global_pass(q, k, v, grid, tile, Hh, out=nanfill.clone())
    torch.cuda.synchronize()
    qq, kk, vv = f64(q), f64(k), f64(v)
    assert maxerr(o1, oracle.local_pass(qq, kk, vv, grid, tile)) <= TOL[dtype]
    assert maxerr(out, oracle.global_pass(qq, kk, vv, grid, tile)) <= TOL[dtype]


def test_cut_forward_halves_compose_and_fill_the_workspace():
    """On a cut tiling the two halves give the forward bit for bit, and the workspace
    holds the local output at every present cell (absent cells are not read)."""
    grid, tile = (5, 12, 20), (2, 5, 6)
    B, Hh, d = 2, 3, 128
    q, k, v = rand_inputs((B, 1200, Hh, d), torch.bfloat16, 23, True)
    out = sq.squad_attn_forward(q, k, v, grid, tile)
    ws = sq.squad_attn_forward_local(q, k, v, grid, tile)
    out2 = sq.squad_attn_forward_global(q, k, grid, tile, ws)
    assert torch.equal(out, out2)
    idx = oracle.padded_window_index(grid, tile)     # [G, Wn], -1 for absent cells
    G, Wn = idx.shape
    o1 = ws.view(torch.float16).reshape(B, Hh, Wn, G, d).transpose(2, 3)   # [B, Hh, G, Wn, d]
    want = oracle.local_pass(f64(q), f64(k), f64(v), grid, tile)           # token order
    present = idx >= 0
    got = f64(o1)[:, :, present]                                           # [B, Hh, n, d] in window order
    exp = np.transpose(want, (0, 2, 1, 3))[:, :, idx[present]]
    assert np.max(np.abs(got - exp)) <= TOL[torch.bfloat16]


def test_cut_forward_on_the_planners_tile():
    """squad_plan_tile's pick for a grid with no whole tiling near sqrt(n) runs and
    matches the oracle."""
    grid = (11, 13, 17)
    tile = sq.squad_plan_tile(grid)
    n = grid[0] * grid[1] * grid[2]
    q, k, v = rand_inputs((1, n, 2, 128), torch.bfloat16, 24)
    say(f"planner tile {grid} -> {tile}")
    out = sq.squad_attn_forward(q, k, v, grid, tile)
    torch.cuda.synchronize()
    assert maxerr(out, oracle.squad_forward(f64(q), f64(k), f64(v), grid, tile)) <= TOL[torch.bfloat16]


def test_mfma_probe_runs_and_is_deterministic():
    """The measuring kernel: finite per-lane checksums, identical across runs."""
    out = torch.empty(8 * 256, dtype=torch.float32, device="cuda")
    sq.squad_debug_mfma_probe(out, 8, 16)
    a = out.clone()
    sq.squad_debug_mfma_probe(out, 8, 16)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all() and torch.equal(a, out)
