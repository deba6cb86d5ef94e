"""GPU parity of the training path (forward_train + backward) against the float64
oracle, through the C ABI."""

import sys

import numpy as np
import pytest
import torch

import oracle
from sub_quadratic_windowed_amd import inputs
import sub_quadratic_windowed_amd as sq

pytestmark = pytest.mark.gpu

# max-abs error of each gradient against the oracle, relative to max(1, max |ref|)
TOL = {torch.float32: 1e-4, torch.bfloat16: 2.5e-2}


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


def rand_case(shape, dtype, seed, peaky=False):
    q, k, v = inputs.make_qkv(shape, dtype, peaky, seed)
    g = torch.Generator().manual_seed(seed + 1000)
    dout = torch.randn(shape, generator=g).to(dtype)
    return tuple(x.cuda() for x in (q, k, v, dout))


def check_grads(got, want, dtype, label):
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        err = float(np.max(np.abs(f64(g) - w)))
        ref = max(1.0, float(np.max(np.abs(w))))
        rms = float(np.sqrt(np.mean((f64(g) - w) ** 2)) / max(1e-30, np.sqrt(np.mean(w ** 2))))
        say(f"  {label} {name}: max-abs {err:.3e} (ref max {ref:.3f}), rel-rms {rms:.3e}")
        assert np.isfinite(f64(g)).all()
        assert err <= TOL[dtype] * ref, (name, err)


BWD_CASES = [
    # grid, tile, batch, heads, head_dim, dtype, peaky
    ((4, 8, 8), (1, 4, 4), 1, 2, 64, torch.float32, False),
    ((4, 6, 10), (2, 3, 5), 2, 3, 128, torch.float32, True),      # W = 30, G = 8: ragged blocks
    ((4, 6, 10), (2, 3, 5), 2, 3, 128, torch.bfloat16, True),
    ((8, 8, 8), (2, 4, 4), 1, 2, 64, torch.bfloat16, False),      # W = 32, G = 16
    ((6, 10, 10), (2, 5, 10), 1, 2, 128, torch.bfloat16, False),  # W = 100, G = 6
    ((8, 12, 10), (1, 12, 10), 1, 2, 128, torch.bfloat16, True),  # W = 120, G = 8
    ((4, 16, 20), (4, 8, 10), 1, 1, 128, torch.bfloat16, False),  # W = 320, G = 4: 3 chunks, 10 blocks
    ((16, 8, 8), (1, 1, 1), 1, 2, 128, torch.bfloat16, False),    # W = 1, G = 1024
    ((4, 8, 8), (4, 8, 8), 1, 2, 64, torch.bfloat16, False),      # G = 1
    ((3, 5, 7), (2, 2, 3), 1, 2, 64, torch.float32, False),       # cut tilings
    ((3, 5, 7), (2, 2, 3), 2, 2, 128, torch.bfloat16, True),
    ((5, 12, 20), (2, 5, 6), 1, 2, 128, torch.bfloat16, False),
    ((4, 8, 8), (1, 8, 8), 1, 2, 128, torch.bfloat16, True),      # W = 64: two-wave workgroups
    ((5, 13, 4), (5, 13, 1), 1, 2, 128, torch.bfloat16, False),   # W = 65: four-wave, one row past
    ((3, 11, 4), (3, 11, 1), 2, 2, 128, torch.bfloat16, True),    # W = 33: a second block of one row
    ((4, 8, 8), (1, 8, 8), 1, 2, 64, torch.float32, False),
    ((5, 13, 20), (4, 12, 12), 1, 2, 128, torch.bfloat16, True),  # cut, Wn = 576 (past the row tables)
    ((9, 31, 40), (2, 2, 2), 1, 2, 128, torch.bfloat16, False),   # cut, G = 1600 (past the row tables)
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: f"{c[0]}-{c[1]}-b{c[2]}h{c[3]}d{c[4]}-{str(c[5])[6:]}")
def test_backward_matches_oracle(case):
    grid, tile, B, Hh, d, dtype, peaky = case
    n = grid[0] * grid[1] * grid[2]
    q, k, v, dout = rand_case((B, n, Hh, d), dtype, 31, peaky)
    say(f"backward {case}")
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    dq, dk, dv = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws)
    torch.cuda.synchronize()
    want = oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), grid, tile)
    check_grads((dq, dk, dv), want, dtype, "")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_backward_with_a_given_scale(dtype):
    grid, tile = (4, 6, 10), (2, 3, 5)
    q, k, v, dout = rand_case((2, 240, 3, 64), dtype, 36, True)
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile, scale=0.3)
    grads = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws, scale=0.3)
    torch.cuda.synchronize()
    want = oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), grid, tile, scale=0.3)
    check_grads(grads, want, dtype, "scale 0.3")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_forward_train_output_and_statistics(dtype):
    """forward_train's output is squad_attn_forward's, bit for bit; the row statistics
    it keeps are each pass's log-sum-exp (log2 domain), unit-major."""
    grid, tile, B, Hh, d = (4, 6, 10), (2, 3, 5), 2, 3, 128
    n = 240
    q, k, v, _ = rand_case((B, n, Hh, d), dtype, 32)
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    ref = sq.squad_attn_forward(q, k, v, grid, tile)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    lse_l, lse_g = oracle.squad_forward_stats(f64(q), f64(k), grid, tile)   # [B, n, Hh], natural log
    G, Wn = 8, 30
    esz = 4 if dtype == torch.float32 else 2
    al = lambda x: (x + 255) // 256 * 256
    bh, cells = B * Hh, G * Wn
    off_l = al(bh * cells * d * esz)
    off_g = al(off_l + bh * cells * 4)
    got_l = ws[off_l:off_l + bh * cells * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    got_g = ws[off_g:off_g + bh * cells * 4].view(torch.float32).cpu().numpy().astype(np.float64)
    idx = oracle.window_index(grid, tile)            # [G, Wn]
    # unit-major: local [G][B*Hh][Wn], global [Wn][B*Hh][G]; unit index s * BH + bh
    want_l = np.empty((G, bh, Wn))
    want_g = np.empty((Wn, bh, G))
    for b in range(B):
        for h in range(Hh):
            want_l[:, b * Hh + h, :] = lse_l[b, idx, h]
            want_g[:, b * Hh + h, :] = lse_g[b, idx.T, h]
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    np.testing.assert_allclose(got_l.reshape(G, bh, Wn), want_l * np.log2(np.e), atol=tol)
    np.testing.assert_allclose(got_g.reshape(Wn, bh, G), want_g * np.log2(np.e), atol=tol)


def test_backward_at_the_5b_dit_shape():
    """The 5B-DiT-shaped workload's per-head shape (grid 32x24x40, tile 2x8x10: W = 160,
    G = 192, d = 128) with 2 heads, every gradient element against the oracle."""
    cfg = inputs.CONFIGS["dit5b_bf16"]
    grid, tile = cfg.grid, cfg.tile
    q, k, v, dout = rand_case((1, cfg.n, 2, 128), torch.bfloat16, 33)
    say("backward dit5b shape, 2 heads")
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    grads = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws)
    torch.cuda.synchronize()
    want = oracle.squad_backward(f64(q), f64(k), f64(v), f64(dout), grid, tile)
    check_grads(grads, want, torch.bfloat16, "dit5b")


def test_autograd_wrapper_matches_the_entry_points():
    grid, tile = (4, 6, 10), (2, 3, 5)
    q, k, v, dout = rand_case((1, 240, 2, 128), torch.bfloat16, 34)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = sq.SquadAttention.apply(qa, ka, va, grid, tile)
    out.backward(dout)
    out2, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    dq, dk, dv = sq.squad_attn_backward(q, k, v, out2, dout, grid, tile, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(qa.grad, dq) and torch.equal(ka.grad, dk) and torch.equal(va.grad, dv)


def test_backward_properties_at_highres_size():
    """Full high-resolution workload (245,760 tokens, 24 heads): the value gradient
    keeps dout's column sums per (batch, head), the key gradient sums to zero, and
    reruns are bit-identical."""
    cfg = inputs.CONFIGS["highres_bf16"]
    q, k, v, dout = rand_case((1, cfg.n, cfg.heads, 128), torch.bfloat16, 35)
    say("backward highres properties")
    out, ws = sq.squad_attn_forward_train(q, k, v, cfg.grid, cfg.tile)
    dq, dk, dv = sq.squad_attn_backward(q, k, v, out, dout, cfg.grid, cfg.tile, ws)
    dq2, dk2, dv2 = sq.squad_attn_backward(q, k, v, out, dout, cfg.grid, cfg.tile, ws)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    for x in (dq, dk, dv):
        assert torch.isfinite(x).all()
    sdv = dv.double().sum(dim=1)
    sdo = dout.double().sum(dim=1)
    scale = dout.double().abs().sum(dim=1)
    # bf16 rounding of each dv element: relative 2^-9, summed over n terms of either sign
    assert float(((sdv - sdo).abs() / scale).max()) < 4e-3
    sdk = dk.double().sum(dim=1)
    assert float((sdk.abs() / dk.double().abs().sum(dim=1)).max()) < 4e-3


def test_training_on_a_side_stream():
    """Forward_train and backward enqueued on a caller's own stream (not torch's
    current one) give the same bits as on the current stream."""
    grid, tile = (4, 6, 10), (2, 3, 5)
    q, k, v, dout = rand_case((1, 240, 2, 128), torch.bfloat16, 37)
    out, ws = sq.squad_attn_forward_train(q, k, v, grid, tile)
    ref = sq.squad_attn_backward(q, k, v, out, dout, grid, tile, ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ws2 = torch.empty_like(ws)
    out2 = torch.empty_like(out)
    grads = [torch.empty_like(q) for _ in range(3)]
    sq.squad_attn_forward_train(q, k, v, grid, tile, out=out2, workspace=ws2, stream=side)
    sq.squad_attn_backward(q, k, v, out2, dout, grid, tile, ws2, dq=grads[0], dk=grads[1], dv=grads[2],
                           stream=side)
    side.synchronize()
    assert torch.equal(out, out2)
    for a, b in zip(ref, grads):
        assert torch.equal(a, b)
