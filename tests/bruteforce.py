"""Brute-force statement of SQuad-Attention as two masked dense attentions.

Independent of the oracle's gather/regroup code: both passes run over all n
tokens in their original order, and the window / offset structure enters only
through n x n boolean masks built from each token's (t, h, w) coordinates.

* local pass  = dense softmax attention with mask [window(i) == window(j)]
  (a block-diagonal mask in window order);
* global pass = dense softmax attention with mask [offset(i) == offset(j)]
  (a strided mask), with v replaced by the local output
  (gist.science technical summary, "1. SQuad-Attention Operator").

float64 numpy only; for tiny inputs (n up to a few hundred).
"""

import numpy as np


def coords(grid):
    T, H, W = grid
    i = np.arange(T * H * W)
    return i // (H * W), (i // W) % H, i % W


def window_id(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    t, h, w = coords(grid)
    # windows of a cut tiling (grid not a whole number of tiles) keep the
    # ceil-sized window grid; absent tokens simply do not occur
    return ((t // tt) * (-(-H // th)) + h // th) * (-(-W // tw)) + w // tw


def offset_id(grid, tile):
    tt, th, tw = tile
    t, h, w = coords(grid)
    return ((t % tt) * th + h % th) * tw + w % tw


def masked_attention_matrix(q, k, mask, scale):
    """A[i, j] = softmax over j with mask[i, j] (float64), for one head: q,k [n, d]."""
    logits = scale * (q @ k.T)
    logits = np.where(mask, logits, -np.inf)
    logits = logits - logits.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(logits), 0.0)
    return e / e.sum(axis=1, keepdims=True)


def local_mask(grid, tile):
    g = window_id(grid, tile)
    return g[:, None] == g[None, :]


def global_mask(grid, tile):
    p = offset_id(grid, tile)
    return p[:, None] == p[None, :]


def matrices(q, k, grid, tile, scale):
    """Per (b, head) local and global attention matrices: A_L, A_G of shape [B, Hh, n, n]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, n, Hh, d = q.shape
    ml, mg = local_mask(grid, tile), global_mask(grid, tile)
    AL = np.empty((B, Hh, n, n))
    AG = np.empty((B, Hh, n, n))
    for b in range(B):
        for h in range(Hh):
            AL[b, h] = masked_attention_matrix(q[b, :, h], k[b, :, h], ml, scale)
            AG[b, h] = masked_attention_matrix(q[b, :, h], k[b, :, h], mg, scale)
    return AL, AG


def squad_bruteforce(q, k, v, grid, tile, scale):
    """out = A_G (A_L v) per (b, head), tokens in original order.  [B, n, Hh, d]."""
    v = np.asarray(v, np.float64)
    AL, AG = matrices(q, k, grid, tile, scale)
    B, n, Hh, d = v.shape
    out = np.empty((B, n, Hh, d))
    o1 = np.empty((B, n, Hh, d))
    for b in range(B):
        for h in range(Hh):
            o1[b, :, h] = AL[b, h] @ v[b, :, h]
            out[b, :, h] = AG[b, h] @ o1[b, :, h]
    return out, o1
