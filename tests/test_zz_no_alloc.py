"""The no-allocation forward against squad_attn_forward, through the C ABI.

squad_attn_forward_noalloc keeps the local output in the library's own per-device
scratch array instead of a caller's workspace, running head slices one after the
other when the whole local output does not fit.  Every slice runs the same kernels
on the same units, so its output must equal squad_attn_forward's bit for bit.
Calls come in pairs, the second on a smaller input, so a second call that read
anything the first one left in the scratch would show.
"""

import sys

import pytest
import torch

from sub_quadratic_windowed_amd import _lib, inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def qkv(shape, dtype, seed, peaky=False):
    return tuple(x.cuda() for x in inputs.make_qkv(shape, dtype, peaky, seed))


def local_bytes(grid, tile, heads, batch, d, dtype):
    return sq.squad_attn_workspace_size(grid, tile, heads, batch, d, dtype)


# pairs of calls: (grid, tile, batch, heads, head_dim, dtype), the second smaller
PAIRS = [
    # 5B-DiT shape at 24 heads: 189 MB of local output, slices of 8 heads; then the
    # small configuration's shape (25 MB, one call)
    (((32, 24, 40), (2, 8, 10), 1, 24, 128, torch.bfloat16), ((16, 16, 16), (1, 8, 8), 1, 24, 128, torch.bfloat16)),
    # batch 2 x 6 heads (94 MB): one slice per batch element; then 2 heads of one
    (((32, 24, 40), (2, 8, 10), 2, 6, 128, torch.bfloat16), ((32, 24, 40), (2, 8, 10), 1, 2, 128, torch.bfloat16)),
    # a cut tiling, then a smaller whole one; fp32
    (((6, 20, 27), (4, 8, 10), 1, 3, 128, torch.bfloat16), ((4, 8, 8), (1, 4, 4), 1, 2, 64, torch.float32)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-b{p[0][2]}h{p[0][3]}-then-{p[1][0]}")
def test_noalloc_equals_the_workspace_forward(pair):
    for i, (grid, tile, B, Hh, d, dtype) in enumerate(pair):
        n = grid[0] * grid[1] * grid[2]
        need = local_bytes(grid, tile, Hh, B, d, dtype)
        say(f"noalloc call {i}: grid {grid} tile {tile} batch {B} heads {Hh} d {d} {dtype}: "
            f"local output {need / 2**20:.1f} MiB (scratch {_lib.NOALLOC_SCRATCH_BYTES / 2**20:.0f} MiB)")
        q, k, v = qkv((B, n, Hh, d), dtype, 40 + i, peaky=True)
        want = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
        out = torch.full_like(q, float("nan"))
        sq.squad_attn_forward_noalloc(q, k, v, grid, tile, Hh, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {i}: max diff {(out.float() - want.float()).abs().max().item()}"


def test_noalloc_at_the_high_resolution_shape():
    """245,760 tokens x 2 heads: one head's local output (62.9 MB) fits the scratch,
    two do not, so the call runs one head at a time; then a smaller call."""
    cfg = inputs.CONFIGS["highres_bf16"]
    q, k, v = qkv((1, cfg.n, 2, 128), torch.bfloat16, 45)
    say("noalloc: high-resolution grid, 2 heads")
    want = sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, 2)
    out = sq.squad_attn_forward_noalloc(q, k, v, cfg.grid, cfg.tile, 2)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    q2, k2, v2 = (x[:, : 4096].contiguous() for x in (q, k, v))
    want2 = sq.squad_attn_forward(q2, k2, v2, (16, 16, 16), (1, 8, 8), 2)
    out2 = sq.squad_attn_forward_noalloc(q2, k2, v2, (16, 16, 16), (1, 8, 8), 2)
    torch.cuda.synchronize()
    assert torch.equal(out2, want2)


def test_noalloc_with_wide_maps():
    """64^3 tokens x 64 heads x 128 = 2^31 elements: the maps are wide, and one head's
    local output (262,144 cells x 256 B = 64 MiB) fills the scratch exactly, so the
    call runs 64 slices of one head; the result equals the workspace forward's."""
    grid, tile, Hh = (64, 64, 64), (4, 8, 8), 64
    gen = torch.Generator(device="cuda").manual_seed(46)
    q, k, v = (torch.randn((1, 64 ** 3, Hh, 128), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    assert 64 ** 3 * 128 * 2 == _lib.NOALLOC_SCRATCH_BYTES
    say("noalloc: wide maps, 64 heads")
    want = sq.squad_attn_forward(q, k, v, grid, tile, Hh)
    out = sq.squad_attn_forward_noalloc(q, k, v, grid, tile, Hh)
    torch.cuda.synchronize()
    assert torch.equal(out, want)
    del q, k, v, out, want
    torch.cuda.empty_cache()


def test_noalloc_rejects_a_head_past_the_scratch():
    grid, tile = (64, 64, 65), (4, 8, 5)   # 266,240 cells x 128 x 2 bytes > 64 MiB
    q = torch.zeros((1, 64 * 64 * 65, 1, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sq.SquadError) as e:
        sq.squad_attn_forward_noalloc(q, q.clone(), q.clone(), grid, tile, 1)
    assert e.value.status == 8
