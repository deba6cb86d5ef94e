"""GPU parity of the attention block (fused QKV projection -> SQuad-Attention ->
output projection) against the float64 oracle, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

import oracle
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

# max-abs error relative to max(1, max |y|)
TOL = {torch.float32: 1e-4, torch.bfloat16: 3e-2}


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


def block_inputs(B, n, hidden, dtype, seed):
    """x ~ N(0, 1); weights ~ N(0, 1/hidden), so q, k, v and y have unit scale."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, n, hidden, generator=g)
    wqkv = torch.randn(3 * hidden, hidden, generator=g) / hidden ** 0.5
    wo = torch.randn(hidden, hidden, generator=g) / hidden ** 0.5
    return tuple(t.to(dtype).cuda() for t in (x, wqkv, wo))


BLOCK_CASES = [
    # grid, tile, batch, heads, head_dim, dtype, dense
    ((4, 6, 10), (2, 3, 5), 2, 2, 64, torch.float32, False),
    ((4, 6, 10), (2, 3, 5), 2, 2, 64, torch.bfloat16, False),
    ((8, 12, 10), (2, 6, 5), 1, 4, 128, torch.bfloat16, False),
    ((3, 5, 7), (2, 2, 3), 1, 2, 128, torch.bfloat16, False),     # cut tiling
    ((4, 8, 8), (1, 4, 4), 1, 2, 128, torch.bfloat16, True),      # dense comparator
    ((4, 8, 8), (1, 4, 4), 1, 2, 64, torch.float32, True),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=lambda c: f"{c[0]}-{c[1]}-h{c[3]}d{c[4]}-{str(c[5])[6:]}-{'dense' if c[6] else 'squad'}")
def test_block_matches_oracle(case):
    grid, tile, B, Hh, d, dtype, dense = case
    n = grid[0] * grid[1] * grid[2]
    x, wqkv, wo = block_inputs(B, n, Hh * d, dtype, 51)
    say(f"block {case}")
    y = sq.squad_block_forward(x, wqkv, wo, grid, tile, Hh, dense=dense)
    torch.cuda.synchronize()
    want = oracle.squad_block_forward(f64(x), f64(wqkv), f64(wo), grid, tile, Hh, dense=dense)
    err = float(np.max(np.abs(f64(y) - want)))
    ref = max(1.0, float(np.max(np.abs(want))))
    say(f"  max-abs {err:.3e} (ref max {ref:.3f})")
    assert np.isfinite(f64(y)).all()
    assert err <= TOL[dtype] * ref


def test_block_at_the_5b_dit_shape_equals_its_parts():
    """The 5B-DiT-shaped block (hidden 3072 = 24 heads x 128, grid 32x24x40, tile
    2x8x10): the fused path (attention reading q, k, v in place from the projection
    rows) equals projection, split into contiguous tensors, squad_attn_forward and
    projection run one by one, to the bf16 rounding of the two paths' outputs."""
    grid, tile, Hh, d = (32, 24, 40), (2, 8, 10), 24, 128
    n, hidden = 30720, 3072
    x, wqkv, wo = block_inputs(1, n, hidden, torch.bfloat16, 52)
    say("block dit5b shape")
    y = sq.squad_block_forward(x, wqkv, wo, grid, tile, Hh)
    qkv = torch.matmul(x[0], wqkv.t().contiguous())                      # [n, 3 hidden]
    q, k, v = (qkv[:, i * hidden:(i + 1) * hidden].contiguous().view(1, n, Hh, d) for i in range(3))
    a = sq.squad_attn_forward(q, k, v, grid, tile)
    y2 = torch.matmul(a.view(n, hidden), wo.t().contiguous())
    torch.cuda.synchronize()
    diff = (y[0].float() - y2.float()).abs()
    say(f"  max |fused - parts| {float(diff.max()):.3e}, mean {float(diff.mean()):.3e}")
    assert torch.isfinite(y).all()
    assert float(diff.max()) <= 3e-2 * max(1.0, float(y2.float().abs().max()))
    assert float(diff.mean()) <= 2e-3


def test_block_on_a_caller_handle():
    """squad_block_forward on a rocBLAS handle the caller creates (squad_blas_create)
    and releases (squad_blas_destroy) gives the same bits as on the binding's own
    handle, also on a side stream."""
    grid, tile, Hh, d = (4, 6, 10), (2, 3, 5), 2, 64
    x, wqkv, wo = block_inputs(1, 240, Hh * d, torch.bfloat16, 53)
    ref = sq.squad_block_forward(x, wqkv, wo, grid, tile, Hh)
    torch.cuda.synchronize()
    h = sq.BlasHandle()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y = torch.empty_like(x)
    sq.squad_block_forward(x, wqkv, wo, grid, tile, Hh, y=y, blas=h, stream=side)
    side.synchronize()
    h.close()
    assert torch.equal(y, ref)
