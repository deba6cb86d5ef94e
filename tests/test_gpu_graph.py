"""The entry points under HIP graph capture: the library enqueues only kernels on
the caller's stream (no allocation, memset or synchronisation inside), so a
captured forward, no-allocation forward, or training forward and backward replays
to the same bits as the eager calls.

Each graph is replayed several times; before every replay new inputs are copied
into the captured input tensors by eager work on the same stream, and every
replay is compared with eager calls on the same inputs.  Outputs, workspaces and
inputs are allocated before capture, so nothing inside the graph allocates.
"""

import sys

import pytest
import torch

from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

REPLAYS = 3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def fresh(shape, dtype, seed, n=3):
    return [x.cuda() for x in inputs.make_qkv(shape, dtype, True, seed)][:n]


CASES = [
    # grid, tile, batch, heads, head_dim, dtype
    ((4, 6, 10), (2, 3, 5), 2, 3, 128, torch.bfloat16),
    ((16, 16, 16), (1, 8, 8), 1, 4, 128, torch.bfloat16),
    ((3, 5, 7), (2, 2, 3), 1, 2, 64, torch.float32),        # cut tiling
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{str(c[5])[6:]}")
def test_forward_replays_match_eager(case):
    grid, tile, B, Hh, d, dtype = case
    n = grid[0] * grid[1] * grid[2]
    shape = (B, n, Hh, d)
    q, k, v = fresh(shape, dtype, 120)
    out = torch.empty_like(q)
    ws = torch.empty(sq.squad_attn_workspace_size(grid, tile, Hh, B, d, dtype), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        sq.squad_attn_forward(q, k, v, grid, tile, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.squad_attn_forward(q, k, v, grid, tile, out=out, workspace=ws)
    for r in range(REPLAYS):
        nq, nk, nv = fresh(shape, dtype, 121 + r)
        q.copy_(nq); k.copy_(nk); v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        want = sq.squad_attn_forward(nq, nk, nv, grid, tile)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"
    say(f"  {case}: {REPLAYS} replays equal to eager")


def test_noalloc_forward_replays_match_eager():
    grid, tile, B, Hh, d, dtype = (16, 16, 16), (1, 8, 8), 1, 4, 128, torch.bfloat16
    shape = (B, 4096, Hh, d)
    q, k, v = fresh(shape, dtype, 130)
    out = torch.empty_like(q)
    sq.squad_attn_forward_noalloc(q, k, v, grid, tile, out=out)   # looks up the scratch array once
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sq.squad_attn_forward_noalloc(q, k, v, grid, tile, out=out)
    for r in range(REPLAYS):
        nq, nk, nv = fresh(shape, dtype, 131 + r)
        q.copy_(nq); k.copy_(nk); v.copy_(nv)
        g.replay()
        torch.cuda.synchronize()
        want = sq.squad_attn_forward(nq, nk, nv, grid, tile)
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"replay {r}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_training_step_replays_match_eager(dtype):
    """forward_train and backward captured in one graph."""
    grid, tile, B, Hh, d = (4, 6, 10), (2, 3, 5), 2, 2, 128
    shape = (B, 240, Hh, d)
    q, k, v = fresh(shape, dtype, 140)
    dout = torch.randn(shape, generator=torch.Generator().manual_seed(141)).to(dtype).cuda()
    out = torch.empty_like(q)
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(sq.squad_attn_train_workspace_size(grid, tile, Hh, B, d, dtype), dtype=torch.uint8,
                     device="cuda")

    def step():
        sq.squad_attn_forward_train(q, k, v, grid, tile, out=out, workspace=ws)
        sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws, dq=grads[0], dk=grads[1], dv=grads[2])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        nq, nk, nv = fresh(shape, dtype, 142 + r)
        nd = torch.randn(shape, generator=torch.Generator().manual_seed(150 + r)).to(dtype).cuda()
        q.copy_(nq); k.copy_(nk); v.copy_(nv); dout.copy_(nd)
        g.replay()
        torch.cuda.synchronize()
        o2, ws2 = sq.squad_attn_forward_train(nq, nk, nv, grid, tile)
        want = sq.squad_attn_backward(nq, nk, nv, o2, nd, grid, tile, ws2)
        torch.cuda.synchronize()
        assert torch.equal(out, o2), f"replay {r}: out"
        for name, a, b in zip(("dq", "dk", "dv"), grads, want):
            assert torch.equal(a, b), f"replay {r}: {name}"
