"""Benchmark: SQuad-Attention forward on one MI355X.

One step = one squad_attn_forward (local pass + global pass, with the window
gather, the window-to-group regroup and the scatter folded into the two kernels'
loads and stores) over the high-resolution workload: batch 1, 24 heads, head_dim
128, latent grid 64x48x80 = 245,760 tokens, tile 4x12x10 (W = 480 tokens per
window, G = 512 windows), bf16 q, k, v drawn i.i.d. N(0, 1) (seed 4), already
resident in HBM when the timed region starts.

Prints one JSON line.  `value` is tokens per second (batch * n / step time).
Beside it: achieved TFLOP/s and the fraction of the bf16 dense MFMA peak, the
roofline object of the dominant kernel (its average duration from HIP events on
the launch stream), the float64 CPU oracle timed on a bounded sample of the same
workload, and a dense full-attention comparator on the 5B-DiT-shaped workload.
Under `tilings`, the same inputs under the planner's compact tile and on a grid
cut by the tiling (one column narrower); under `backward`, the training path
(forward keeping its statistics, then the gradients) on the same inputs; under
`kpass`, the three-level operator on the same inputs; under `block`, the
attention block (projections, attention, output projection) at the 5B-DiT shape
with SQuad and with dense attention.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 (256 CU x 2.4 GHz x 4096 flop/clk)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
METRIC = "SQuad-attn tokens/s and TFLOP/s (% bf16 MFMA peak) at 1 MI355X"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="highres_bf16")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-dense", action="store_true")
    p.add_argument("--no-permutations", action="store_true")
    p.add_argument("--no-tilings", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=0,
                   help="heads in the oracle's timed run (default: all of the workload's heads)")
    return p.parse_args()


# the sources each kernel family is built from (its kernel file, the shared maps and
# launch interface, and the host code that sets up its arguments)
KERNEL_SOURCES = {
    "forward": ("attn_bf16.hip",),
    "backward": ("attn_bwd_bf16.hip",),
    "permute": ("permute.hip",),
}
SHARED_SOURCES = ("squad_map.h", "squad_kernels.h", "squad_api.hip")


def kernel_source_digest(family="forward"):
    """Digest of the sources of one kernel family: counters taken on other sources
    do not describe the kernels that run."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family] + SHARED_SOURCES:
        with open(os.path.join(ROOT, "sub_quadratic_windowed_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, digest):
    """HBM bytes per launch measured by rocprofv3 counters for this kernel source, if any."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, stream, iters):
    """Average duration (ms) of fn() over iters launches, from HIP events on `stream`."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def cold_and_copy(step, stream, dev, calls=20):
    """Per-call forward times with the 256 MB last-level cache cleared first (a 1 GiB
    scrub buffer written between calls, outside the timed region), median and min;
    and the bandwidth of a plain 1 GiB device copy on the same card."""
    import torch

    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for i in range(calls):
        scrub.fill_(i & 0xff)
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    dst = torch.empty_like(scrub)
    dst.copy_(scrub)
    torch.cuda.synchronize()
    copy_ms = time_launches(lambda: dst.copy_(scrub), stream, 10)
    del scrub, dst
    return {"cold_median_ms": round(ms[len(ms) // 2], 4), "cold_min_ms": round(ms[0], 4), "calls": calls,
            "copy_1gib_gbs": round(2.0 * (1 << 30) / copy_ms / 1e6, 1)}


def mfma_probe(sq, stream, dev):
    """The card's sustained bf16 MFMA rate with random operands (the library's
    measuring kernel: nothing but independent 32x32x16 MFMA chains)."""
    import torch

    blocks, iters = 2048, 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    run = lambda: sq.squad_debug_mfma_probe(out, blocks, iters, stream=stream)
    run()
    torch.cuda.synchronize()
    ms = time_launches(run, stream, 5)
    flops = blocks * 4.0 * iters * 4 * 32768.0
    del out
    return {"tflops": round(flops / ms / 1e9, 1), "frac_of_peak": round(flops / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
            "kernel": "4 independent 32x32x16 bf16 MFMA chains per wave, hash-drawn operands, 8192 waves"}


def cpu_baseline(cfg, qc, kc, vc, heads, chunk=8):
    """The float64 oracle as it stands, timed over `heads` of the workload's heads
    (all of them by default).  Heads are independent, so it runs `chunk` heads per
    call to bound its memory (at the high-resolution size one call over 8 heads
    holds about 25 GB); the time is the sum over the calls."""
    import threadpoolctl

    import oracle

    heads = heads or cfg.heads
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    dt = 0.0
    calls = 0
    for h0 in range(0, heads, chunk):
        hs = list(range(h0, min(h0 + chunk, heads)))
        q = qc[:, :, hs].double().numpy()
        k = kc[:, :, hs].double().numpy()
        v = vc[:, :, hs].double().numpy()
        t0 = time.perf_counter()
        oracle.squad_forward(q, k, v, cfg.grid, cfg.tile)
        dt += time.perf_counter() - t0
        calls += 1
        del q, k, v
    # tokens/s of the whole workload (scaled only if fewer than all heads ran)
    value = cfg.batch * cfg.n * (heads / cfg.heads) / dt
    scaled = "" if heads == cfg.heads else f", scaled by {cfg.heads}/{heads} to the whole workload"
    return {
        "value": value,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 numpy oracle, full forward over {heads} of {cfg.heads} heads "
                  f"({cfg.batch}x{cfg.n} tokens, head_dim {cfg.head_dim}) in {calls} calls of up to "
                  f"{chunk} heads; {dt:.1f} s{scaled}",
        "seconds": dt,
        "blas_threads": threads,
        "affinity_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family, model and
    stepping numbers, and the logical CPU count; or None."""
    fields, count = {}, 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                key, _, val = line.partition(":")
                key = key.strip()
                if key == "processor":
                    count += 1
                elif key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                    fields[key] = val.strip()
    except OSError:
        return None
    if "model name" not in fields:
        return None
    return (f"{fields['model name']} (family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}, "
            f"stepping {fields.get('stepping', '?')}), {count} logical CPUs")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the heads of SQuad-Attention "
              "shard across GPUs with no exchange, so N GPUs would each run this workload's heads/N.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sub_quadratic_windowed_amd as sq
    from sub_quadratic_windowed_amd import inputs

    cfg = inputs.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    qc, kc, vc = inputs.config_inputs(cfg)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(sq.squad_attn_workspace_size(cfg.grid, cfg.tile, cfg.heads, cfg.batch, cfg.head_dim,
                                                  cfg.dtype), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads, out=out, workspace=ws, stream=stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    print(f"[bench] {args.steps} steps, {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # ---- per-kernel durations: each half of the forward alone, HIP events on the launch stream
    local = lambda: sq.squad_attn_forward_local(q, k, v, cfg.grid, cfg.tile, cfg.heads, workspace=ws,
                                                stream=stream)
    glob = lambda: sq.squad_attn_forward_global(q, k, cfg.grid, cfg.tile, ws, cfg.heads, out=out, stream=stream)
    iters = max(args.steps, 10)
    ms_local = time_launches(local, stream, iters)
    ms_global = time_launches(glob, stream, iters)
    ms_fwd = time_launches(step, stream, iters)

    B, n, H, d, W, G = cfg.batch, cfg.n, cfg.heads, cfg.head_dim, cfg.window, cfg.windows
    rows = B * n * H                                   # (token, head) rows
    flops_local = 4.0 * d * W * rows                   # QK^T and PV of the local pass
    flops_global = 4.0 * d * G * rows
    flops = flops_local + flops_global
    bytes_per_pass = 8.0 * d * rows                    # read q, k, v (or o1), write o1 (or out): 4 x d x 2 B
    tokens_per_s = B * n / (ms_per_step * 1e-3)
    tflops = flops / (ms_per_step * 1e-3) / 1e12

    kernels = {
        "local": {"ms": ms_local, "tflops": flops_local / ms_local / 1e9,
                  "gbs": bytes_per_pass / ms_local / 1e6},
        "global": {"ms": ms_global, "tflops": flops_global / ms_global / 1e9,
                   "gbs": bytes_per_pass / ms_global / 1e6},
        "forward_events_ms": ms_fwd,
    }
    dom = "local" if ms_local >= ms_global else "global"
    dom_name = {"local": "attn16_kernel<128,4,bf16,fp16> (local pass)",
                "global": "attn16_kernel<128,4,fp16,bf16> (global pass)"}[dom]
    achieved = kernels[dom]["gbs"]
    digest = kernel_source_digest()
    traffic = traffic_from_profiles(dom, digest)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "kernel": dom_name,
        "algorithmic_bytes_per_launch": bytes_per_pass,
        "mfma_tflops": round(kernels[dom]["tflops"], 1),
        "mfma_frac": round(kernels[dom]["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
        "source_digest": digest,
    }

    print("[bench] cold-cache forward and copy bandwidth", file=sys.stderr, flush=True)
    cold = cold_and_copy(step, stream, dev)
    probe = mfma_probe(sq, stream, dev)
    roofline["measured_mfma_tflops"] = probe["tflops"]
    roofline["mfma_frac_of_measured"] = round(kernels[dom]["tflops"] / probe["tflops"], 4)

    perms = None
    if not args.no_permutations:
        perms = permutation_rates(sq, cfg, q, stream)

    backward = None
    if not args.no_backward:
        print("[bench] training path (forward_train + backward)", file=sys.stderr, flush=True)
        backward = backward_rates(sq, cfg, q, k, v, stream)

    kpass = None
    if not args.no_tilings and cfg.name == "highres_bf16":
        print("[bench] three-level operator", file=sys.stderr, flush=True)
        kpass = kpass_rates(sq, q, k, v, H, stream)

    tilings = None
    if not args.no_tilings and cfg.name == "highres_bf16":
        print("[bench] other tilings of the workload", file=sys.stderr, flush=True)
        tilings = tiling_rates(sq, q, k, v, H, stream)

    dense = None
    if not args.no_dense:
        del out, ws
        torch.cuda.empty_cache()
        dense = dense_comparator(sq, inputs, dev)

    block = None
    if not args.no_dense:
        block = block_rates(sq, inputs, dev)

    graphs = None
    if not args.no_dense:
        print("[bench] graph replays of the small configurations", file=sys.stderr, flush=True)
        try:
            graphs = graph_rates(sq, inputs, dev)
        except Exception as e:   # reported, not fatal: the headline line still prints
            graphs = {"error": f"{type(e).__name__}: {e}"}

    base = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu oracle on {args.cpu_heads or cfg.heads} heads", file=sys.stderr, flush=True)
        base = cpu_baseline(cfg, qc, kc, vc, args.cpu_heads)
        base["gpu_over_cpu"] = round(tokens_per_s / base["value"], 1)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: batch {B}, {H} heads, head_dim {d}, grid {'x'.join(map(str, cfg.grid))}, "
                        f"tile {'x'.join(map(str, cfg.tile))} (W={W}, G={G}), q,k,v iid N(0,1) bf16",
            "batch": B, "tokens": n, "heads": H, "head_dim": d,
            "grid": list(cfg.grid), "tile": list(cfg.tile), "parallelism": "none (1 GPU)",
        },
        "tflops": round(tflops, 1),
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        # against min(MFMA peak, intensity x HBM peak), intensity = flops / (8 tensor passes)
        "pct_roofline": round(100 * tflops / min(MFMA_BF16_PEAK_TFLOPS,
                                                  flops / (2 * bytes_per_pass) * HBM_PEAK_GBS / 1e3), 2),
        "cold": cold,
        "mfma_probe": probe,
        "flops_per_step": flops,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": base,
        "dense_comparator": dense,
        "permutations": perms,
        "tilings": tilings,
        "backward": backward,
        "kpass": kpass,
        "block": block,
        "graph": graphs,
    }
    print(json.dumps(line), flush=True)


def graph_rates(sq, inputs, dev, iters=200):
    """The forward of the two smallest configurations called eagerly through the
    binding, back to back, against the same forward captured once in a HIP graph
    and replayed: per-call time (ms) from HIP events.  With kernels of a few
    microseconds the eager calls are bound by the host (argument checks, two
    launches); a replay issues both kernels at once.  The replayed output equals
    the eager one bit for bit."""
    import torch

    res = {}
    for name in ("tiny_fp32", "small_bf16"):
        cfg = inputs.CONFIGS[name]
        q, k, v = (x.to(dev) for x in inputs.config_inputs(cfg))
        out = torch.empty_like(q)
        ws = torch.empty(sq.squad_attn_workspace_size(cfg.grid, cfg.tile, cfg.heads, cfg.batch, cfg.head_dim,
                                                      cfg.dtype), dtype=torch.uint8, device=dev)

        def fwd():
            sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads, out=out, workspace=ws)

        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            for _ in range(3):
                fwd()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fwd()
        stream = torch.cuda.current_stream(dev)
        fwd()
        torch.cuda.synchronize()
        ref = out.clone()
        eager = time_launches(fwd, stream, iters)
        replay = time_launches(g.replay, stream, iters)
        torch.cuda.synchronize()
        res[name] = {"eager_ms": round(eager, 4), "graph_replay_ms": round(replay, 4),
                     "replay_equals_eager": bool(torch.equal(out, ref))}
        del g
    return res


def permutation_rates(sq, cfg, q, stream):
    """GB/s (read + write bytes / HIP-event time) of the standalone reshaping kernels
    on the workload's q tensor: tile gather, window-to-group regroup, tile scatter."""
    import torch

    B, n, H, d, W, G = cfg.batch, cfg.n, cfg.heads, cfg.head_dim, cfg.window, cfg.windows
    win = torch.empty((B, H, G, W, d), dtype=q.dtype, device=q.device)
    grp = torch.empty((B, H, W, G, d), dtype=q.dtype, device=q.device)
    tok = torch.empty_like(q)
    nbytes = 2.0 * q.numel() * q.element_size()
    runs = {
        "tile_gather": lambda: sq.squad_tile_gather(q, cfg.grid, cfg.tile, dst=win, stream=stream),
        "window_to_group": lambda: sq.squad_window_to_group(win, cfg.grid, cfg.tile, dst=grp, stream=stream),
        "tile_scatter": lambda: sq.squad_tile_scatter(win, cfg.grid, cfg.tile, dst=tok, stream=stream),
    }
    out = {}
    for name, fn in runs.items():
        fn()
        torch.cuda.synchronize()
        ms = time_launches(fn, stream, 10)
        out[name] = {"ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                     "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4)}
    del win, grp, tok
    return out


def backward_rates(sq, cfg, q, k, v, stream):
    """The training path on the workload's inputs: squad_attn_forward_train, then
    squad_attn_backward with a seeded upstream gradient, each timed alone with HIP
    events.  TFLOP/s counts the standard 2.5x-forward work of a softmax-attention
    backward (five products of 2 d L flops per row and pass: S, dP, dV, dK, dQ);
    the kernels compute S and dP twice (once per kind), seven products."""
    import torch

    g = torch.Generator(device=q.device).manual_seed(77)
    dout = torch.randn(q.shape, generator=g, device=q.device, dtype=torch.float32).to(q.dtype)
    out = torch.empty_like(q)
    ws = torch.empty(sq.squad_attn_train_workspace_size(cfg.grid, cfg.tile, cfg.heads, cfg.batch, cfg.head_dim,
                                                        cfg.dtype), dtype=torch.uint8, device=q.device)
    grads = [torch.empty_like(q) for _ in range(3)]
    fwd = lambda: sq.squad_attn_forward_train(q, k, v, cfg.grid, cfg.tile, cfg.heads, out=out, workspace=ws,
                                              stream=stream)
    bwd = lambda: sq.squad_attn_backward(q, k, v, out, dout, cfg.grid, cfg.tile, ws, cfg.heads, dq=grads[0],
                                         dk=grads[1], dv=grads[2], stream=stream)
    fwd()
    bwd()
    torch.cuda.synchronize()
    ms_f = time_launches(fwd, stream, 10)
    ms_b = time_launches(bwd, stream, 10)
    rows = cfg.batch * cfg.n * cfg.heads
    flops = 10.0 * cfg.head_dim * (cfg.window + cfg.windows) * rows
    del ws, grads, out, dout
    return {"forward_train_ms": round(ms_f, 4), "backward_ms": round(ms_b, 4),
            "backward_tflops": round(flops / ms_b / 1e9, 1),
            "backward_flops": flops, "train_step_ms": round(ms_f + ms_b, 4)}


def kpass_rates(sq, q, k, v, heads, stream):
    """The three-level operator over the high-resolution grid: nested tiles 4x4x4 |
    16x16x16 | 64x48x80, units of 64, 64 and 60 tokens (about n^(1/3) each), on the
    workload's inputs; beside the two-pass forward it does 188 / 992 of the work."""
    import torch

    grid, tiles = (64, 48, 80), [(4, 4, 4), (16, 16, 16)]
    out = torch.empty_like(q)
    ws = torch.empty(sq.squad_kpass_workspace_size(grid, tiles, heads, 1, q.shape[-1], q.dtype),
                     dtype=torch.uint8, device=q.device)
    fwd = lambda: sq.squad_kpass_forward(q, k, v, grid, tiles, heads, out=out, workspace=ws, stream=stream)
    fwd()
    torch.cuda.synchronize()
    ms = time_launches(fwd, stream, 20)
    n = grid[0] * grid[1] * grid[2]
    flops = 4.0 * q.shape[-1] * (64 + 64 + 60) * n * heads
    del ws
    # training: the forward keeping its state, then the gradients
    tws = torch.empty(sq.squad_kpass_train_workspace_size(grid, tiles, heads, 1, q.shape[-1], q.dtype),
                      dtype=torch.uint8, device=q.device)
    dout = torch.randn(q.shape, generator=torch.Generator(device=q.device).manual_seed(78), device=q.device,
                       dtype=torch.float32).to(q.dtype)
    grads = [torch.empty_like(q) for _ in range(3)]
    ftrain = lambda: sq.squad_kpass_forward_train(q, k, v, grid, tiles, heads, out=out, workspace=tws, stream=stream)
    bwd = lambda: sq.squad_kpass_backward(q, k, v, out, dout, grid, tiles, tws, heads, dq=grads[0], dk=grads[1],
                                          dv=grads[2], stream=stream)
    ftrain()
    bwd()
    torch.cuda.synchronize()
    ms_ft = time_launches(ftrain, stream, 10)
    ms_b = time_launches(bwd, stream, 10)
    del out, tws, dout, grads
    return {"grid": list(grid), "tiles": [list(t) for t in tiles], "levels": 3, "unit_rows": [64, 64, 60],
            "ms": round(ms, 4), "tokens_per_s": round(n / (ms * 1e-3), 1), "tflops": round(flops / ms / 1e9, 1),
            "forward_train_ms": round(ms_ft, 4), "backward_ms": round(ms_b, 4)}


def present_pairs(grid, tile):
    """(sum over windows of present^2, sum over offset groups of present^2): the
    query-key pairs of the two passes on a possibly cut tiling.  Separable by axis:
    a window's present count is the product of its per-axis extents, an offset
    group's the product of per-axis counts of windows that reach that offset."""
    win = grp = 1
    for X, t in zip(grid, tile):
        k = -(-X // t)
        ext = [t] * (k - 1) + [X - t * (k - 1)]
        win *= sum(e * e for e in ext)
        grp *= sum(sum(1 for e in ext if e > a) ** 2 for a in range(t))
    return win, grp


def tiling_rates(sq, q, k, v, heads, stream):
    """Forward time on the workload's inputs under two more tilings of the same
    window size: the compact tile the planner picks for the grid (whole), and the
    grid one column narrower (64 x 48 x 79: the last column of windows is cut to 9
    of 10 cells, so every global group of offsets w = 9 loses one row)."""
    import torch

    d = q.shape[-1]
    out = {}
    for name, grid, tile in (("whole_planner", (64, 48, 80), tuple(sq.squad_plan_tile((64, 48, 80)))),
                             ("cut_w", (64, 48, 79), (8, 6, 10))):
        n = grid[0] * grid[1] * grid[2]
        qs, ks, vs = q[:, :n], k[:, :n], v[:, :n]     # the first n tokens (batch 1: contiguous)
        o = torch.empty_like(qs)
        ws = torch.empty(sq.squad_attn_workspace_size(grid, tile, heads, 1, d, qs.dtype), dtype=torch.uint8,
                         device=q.device)
        fwd = lambda: sq.squad_attn_forward(qs, ks, vs, grid, tile, heads, out=o, workspace=ws, stream=stream)
        fwd()
        torch.cuda.synchronize()
        ms = time_launches(fwd, stream, 20)
        pw, pg = present_pairs(grid, tile)
        flops = 4.0 * d * heads * (pw + pg)
        out[name] = {"grid": list(grid), "tile": list(tile), "ms": round(ms, 4),
                     "tokens_per_s": round(n / (ms * 1e-3), 1), "tflops": round(flops / ms / 1e9, 1)}
        del o, ws
    return out


def block_rates(sq, inputs, dev):
    """The attention block at the 5B-DiT shape (hidden 3072 = 24 heads x 128, grid
    32x24x40, tile 2x8x10): x -> fused QKV projection -> attention -> output
    projection, with SQuad-Attention and with dense attention (the comparator).
    Synthetic weights, N(0, 1/hidden)."""
    import torch

    cfg = inputs.CONFIGS["dit5b_bf16"]
    hidden = cfg.heads * cfg.head_dim
    g = torch.Generator(device=dev).manual_seed(90)
    x = torch.randn(1, cfg.n, hidden, generator=g, device=dev).to(torch.bfloat16)
    wqkv = (torch.randn(3 * hidden, hidden, generator=g, device=dev) / hidden ** 0.5).to(torch.bfloat16)
    wo = (torch.randn(hidden, hidden, generator=g, device=dev) / hidden ** 0.5).to(torch.bfloat16)
    y = torch.empty_like(x)
    ws = torch.empty(sq.squad_block_workspace_size(cfg.grid, cfg.tile, cfg.heads, 1, cfg.head_dim, torch.bfloat16),
                     dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    run = lambda dense: sq.squad_block_forward(x, wqkv, wo, cfg.grid, cfg.tile, cfg.heads, y=y, dense=dense,
                                               workspace=ws, stream=s)
    run(False)
    run(True)
    torch.cuda.synchronize()
    ms_sq = time_launches(lambda: run(False), s, 20)
    ms_dense = time_launches(lambda: run(True), s, 5)
    gemm_flops = 2.0 * cfg.n * hidden * 4 * hidden
    attn_sq = 4.0 * cfg.head_dim * (cfg.window + cfg.windows) * cfg.n * cfg.heads
    attn_dense = 4.0 * cfg.head_dim * cfg.n * cfg.n * cfg.heads
    del x, y, ws
    return {"workload": f"{cfg.name} block: hidden {hidden}, grid {'x'.join(map(str, cfg.grid))}, "
                        f"tile {'x'.join(map(str, cfg.tile))}",
            "squad_block_ms": round(ms_sq, 4), "dense_block_ms": round(ms_dense, 4),
            "latency_ratio": round(ms_dense / ms_sq, 2),
            "projection_gflop": round(gemm_flops / 1e9, 1),
            "squad_block_tflops": round((gemm_flops + attn_sq) / ms_sq / 1e9, 1),
            "dense_block_tflops": round((gemm_flops + attn_dense) / ms_dense / 1e9, 1)}


def dense_pair(sq, inputs, dev, name, dense_iters):
    """SQuad forward vs dense full attention on one configuration's inputs."""
    import torch

    cfg = inputs.CONFIGS[name]
    print(f"[bench] dense comparator on {name}", file=sys.stderr, flush=True)
    qc, kc, vc = inputs.config_inputs(cfg)
    q, k, v = qc.to(dev), kc.to(dev), vc.to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(sq.squad_attn_workspace_size(cfg.grid, cfg.tile, cfg.heads, 1, 128, cfg.dtype),
                     dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    fwd = lambda: sq.squad_attn_forward(q, k, v, cfg.grid, cfg.tile, cfg.heads, out=out, workspace=ws, stream=s)
    dense = lambda: sq.squad_dense_attn_forward(q, k, v, out=out, stream=s)
    for f in (fwd, dense):
        f()
    torch.cuda.synchronize()
    ms_sq = time_launches(fwd, s, 20)
    ms_dense = time_launches(dense, s, dense_iters)
    n, H, d, W, G = cfg.n, cfg.heads, cfg.head_dim, cfg.window, cfg.windows
    f_sq = 4.0 * d * (W + G) * n * H
    f_dense = 4.0 * d * n * n * H
    del q, k, v, out, ws
    return {
        "workload": f"{cfg.name}: grid {'x'.join(map(str, cfg.grid))}, tile {'x'.join(map(str, cfg.tile))}, "
                    f"{H} heads, head_dim {d}",
        "squad_ms": round(ms_sq, 4),
        "dense_ms": round(ms_dense, 4),
        "latency_ratio": round(ms_dense / ms_sq, 2),
        "flop_ratio": round(f_dense / f_sq, 2),
        "dense_tflops": round(f_dense / ms_dense / 1e9, 1),
        "squad_tflops": round(f_sq / ms_sq / 1e9, 1),
    }


def dense_comparator(sq, inputs, dev):
    """SQuad forward vs dense full attention: the 5B-DiT-shaped workload, plus the
    small and the longer-clip configurations under `other_configs`."""
    line = dense_pair(sq, inputs, dev, "dit5b_bf16", 5)
    line["other_configs"] = [dense_pair(sq, inputs, dev, "small_bf16", 20),
                             dense_pair(sq, inputs, dev, "long_bf16", 3)]
    return line


if __name__ == "__main__":
    main()
