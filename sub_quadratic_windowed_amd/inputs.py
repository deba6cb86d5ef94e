"""Seeded synthetic inputs for SQuad-Attention, shared by the tests, the benchmark
and the smoke check.  Holds no arithmetic of the method: it only draws q, k, v.

The pages measure on Wan 2.2 5B text-to-video latents whose shapes they never
give; these configurations stand in for them.  The "peaky" draws scale each
(batch, token, head) row of q and k by an independent U(0.5, 2) factor so that
softmax rows concentrate on few keys, the structure the pages describe (most
token links weak, a small group strong).
"""

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple
    tile: tuple
    dtype: torch.dtype
    peaky: bool
    seed: int

    @property
    def n(self):
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def window(self):
        return self.tile[0] * self.tile[1] * self.tile[2]

    @property
    def windows(self):
        return self.n // self.window

    @property
    def shape(self):
        return (self.batch, self.n, self.heads, self.head_dim)


CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 1, 2, 64, (4, 8, 8), (1, 4, 4), torch.float32, False, 0),
    "small_bf16": Config("small_bf16", 1, 24, 128, (16, 16, 16), (1, 8, 8), torch.bfloat16, True, 1),
    "dit5b_bf16": Config("dit5b_bf16", 1, 24, 128, (32, 24, 40), (2, 8, 10), torch.bfloat16, False, 2),
    "long_bf16": Config("long_bf16", 1, 24, 128, (64, 32, 32), (4, 8, 8), torch.bfloat16, True, 3),
    "highres_bf16": Config("highres_bf16", 1, 24, 128, (64, 48, 80), (4, 12, 10), torch.bfloat16, False, 4),
}


def make_qkv(shape, dtype, peaky, seed):
    """q, k, v as CPU tensors of `dtype`: i.i.d. N(0,1) fp32 draws (q, then k, then v),
    then for peaky inputs one U(0.5, 2) factor per row of q and of k (drawn after v),
    then a round-to-nearest-even cast."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x)
    if peaky:
        row = tuple(shape[:-1]) + (1,)
        uq = torch.empty(row, dtype=torch.float32).uniform_(0.5, 2.0, generator=g)
        uk = torch.empty(row, dtype=torch.float32).uniform_(0.5, 2.0, generator=g)
        out[0].mul_(uq)
        out[1].mul_(uk)
    return tuple(x.to(dtype) for x in out)


def config_inputs(cfg, seed=None):
    """The seeded q, k, v of a configuration (CPU tensors)."""
    return make_qkv(cfg.shape, cfg.dtype, cfg.peaky, cfg.seed if seed is None else seed)
