"""Oracle for SQuad-Attention: a plain, slow, float64 CPU statement of the operator.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

What is computed, and where the pages define it
-----------------------------------------------
Source pages (all titled "SQuad: Sub-Quadratic Attention Distillation for Efficient
Video Generation"):

* gist.science, technical summary ("Technische Samenvatting"), section
  "Methodologie: SQuad", item "1. SQuad-Attention Operator":
    - Local Pass Attn_L: tokens mix inside fixed windows of size w.
    - Global Pass Attn_G: tokens that sit at the same relative position inside
      their window mix across all windows.
    - Composition: the local pass's output is the value stream of the global pass.
    - Complexity: w = sqrt(n) gives O(n sqrt n); both passes use the standard
      softmax.
* the abstract (arxivdaily.com and the arXiv listing): self-attention over the n
  latent tokens of a video DiT, softmax(QK^T); the distilled attention has no
  extra learnable parameters (gist.science, "Experimentele Resultaten").

Readings taken where the pages are silent (each one is also listed in the design
notes of this repository):

* Tokens are the cells of a T x H x W latent grid, flattened row-major over
  (t, h, w).  A window is a tt x th x tw tile of that grid.  Windows are numbered
  row-major over the window grid (ceil(T/tt), ceil(H/th), ceil(W/tw)); the
  relative position (offset) of a token inside its window is numbered row-major
  over (tt, th, tw).  Only the partitions matter: attention is
  permutation-equivariant inside a window and inside an offset group.
* A grid that is not a whole number of tiles is read as padded up to one with
  absent tokens: the tiles along the far edges are cut by the grid, so their
  windows hold fewer tokens, and an offset group holds one token per window that
  has a token at that offset.  Absent tokens are neither keys nor queries (the
  pages only use whole tiles; this is the plainest extension, and on a whole
  number of tiles it is the operator above).
* The global pass uses the same q and k as the local pass (there are no extra
  parameters), with v replaced by the local output; out = Attn_G(q, k, Attn_L(q, k, v)).
  Nothing is added to it (no residual, gate or sum).
* Softmax scale s = 1/sqrt(d) in both passes unless the caller gives another;
  softmax is taken in its max-subtracted form.
* Batch elements and heads are independent; there is no mask and no causality.

Gradients (squad_backward and the per-pass backwards) are the chain rule applied
to the definitions above: the pages state no gradient formula, but the distillation
they run (flow-matching SFT, then DMD2; technical summary, "Methodologie") trains
through the operator.  q and k receive the sum of both passes' gradients; the
global pass's value gradient is the upstream gradient of the local output.
squad_forward_stats gives each row's softmax normaliser (log-sum-exp) per pass.

More than two passes (squad_kpass_forward): the pages name composing more than
two passes as future work.  The reading taken: nested tiles t1 | t2 | ... | grid
split each axis coordinate into k digits; pass j attends among the tokens that
differ only in digit j, and each pass's output is the next pass's value stream.
k = 2 is the operator above.  squad_kpass_backward is its chain rule over the
levels.

All arithmetic is float64.  Every function below is written from the definition,
with numpy fancy indexing and numpy matmul as its only library steps.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "is_whole",
    "padded_window_index",
    "window_index",
    "softmax_attention",
    "local_pass",
    "global_pass",
    "squad_forward",
    "squad_forward_groups",
    "dense_attention",
    "tile_gather",
    "tile_scatter",
    "window_to_group",
    "window_attn",
    "softmax_attention_backward",
    "local_pass_backward",
    "global_pass_backward",
    "squad_backward",
    "squad_forward_stats",
    "kpass_level_index",
    "squad_kpass_forward",
    "squad_kpass_backward",
    "squad_block_forward",
]


def _check_grid(grid, tile, partial=False):
    T, H, W = (int(x) for x in grid)
    tt, th, tw = (int(x) for x in tile)
    if min(T, H, W, tt, th, tw) <= 0:
        raise ValueError("grid and tile sizes must be positive")
    if tt > T or th > H or tw > W:
        raise ValueError(f"tile {tile} is larger than grid {grid}")
    if not partial and (T % tt or H % th or W % tw):
        raise ValueError(f"grid {grid} is not a whole number of {tile} tiles")
    return T, H, W, tt, th, tw


def is_whole(grid, tile) -> bool:
    """True when the grid is a whole number of tiles."""
    return all(int(x) % int(y) == 0 for x, y in zip(grid, tile))


def padded_window_index(grid, tile) -> np.ndarray:
    """Token index of every (window, offset) pair of a possibly cut tiling.

    idx[g, p] is the token at offset p of window g, or -1 where the tile reaches
    past the grid; windows run row-major over (ceil(T/tt), ceil(H/th), ceil(W/tw)).
    On a whole number of tiles this equals window_index.
    """
    T, H, W, tt, th, tw = _check_grid(grid, tile, partial=True)
    nt, nh, nw = -(-T // tt), -(-H // th), -(-W // tw)
    gt, gh, gw, at, ah, aw = np.ix_(np.arange(nt), np.arange(nh), np.arange(nw),
                                    np.arange(tt), np.arange(th), np.arange(tw))
    t, h, w = gt * tt + at, gh * th + ah, gw * tw + aw
    idx = np.where((t < T) & (h < H) & (w < W), (t * H + h) * W + w, -1)
    return idx.reshape(nt * nh * nw, tt * th * tw)


def window_index(grid, tile) -> np.ndarray:
    """Token index of every (window, offset) pair: an int64 array idx[G, Wn].

    idx[g, p] is the row-major (t, h, w) token index of the token at relative
    position p inside window g.  Windows are the "fixed windows of size w" of the
    local pass; row p of idx.T is the set of tokens "at the same relative position
    within each window" that the global pass mixes (gist.science technical
    summary, Methodologie, "1. SQuad-Attention Operator").
    """
    T, H, W, tt, th, tw = _check_grid(grid, tile)
    tok = np.arange(T * H * W, dtype=np.int64).reshape(T, H, W)
    # split each axis into (window coordinate, coordinate inside the window)
    tok = tok.reshape(T // tt, tt, H // th, th, W // tw, tw)
    # windows row-major over (T/tt, H/th, W/tw), offsets row-major over (tt, th, tw)
    tok = tok.transpose(0, 2, 4, 1, 3, 5)
    return tok.reshape((T // tt) * (H // th) * (W // tw), tt * th * tw).copy()


def softmax_attention(q, k, v, scale) -> np.ndarray:
    """Standard softmax attention over the last two axes, in float64.

    q: [..., Lq, d], k: [..., Lk, d], v: [..., Lk, dv].  Row i of the result is
    sum_j a_ij v_j with a_ij = exp(l_ij - max_j l_ij) / sum_j exp(l_ij - max_j l_ij)
    and l_ij = scale * <q_i, k_j>.  Both passes of the operator use this standard
    softmax (gist.science technical summary, "1. SQuad-Attention Operator",
    Complexiteit).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    logits = logits - logits.max(axis=-1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=-1, keepdims=True)
    return np.matmul(w, v)


def _default_scale(d, scale):
    return 1.0 / np.sqrt(d) if scale is None or scale <= 0 else float(scale)


def _as_bnhd(x, name):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 4:
        raise ValueError(f"{name} must be [batch, n, heads, head_dim]")
    return x


def local_pass(q, k, v, grid, tile, scale=None) -> np.ndarray:
    """Attn_L: softmax attention inside each window.  [B, n, Hh, d] -> [B, n, Hh, d].

    gist.science technical summary, "1. SQuad-Attention Operator", Local Pass.
    """
    q, k, v = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v")))
    s = _default_scale(q.shape[-1], scale)
    if not is_whole(grid, tile):
        return _unit_attention(q, k, v, padded_window_index(grid, tile), s)
    idx = window_index(grid, tile)                      # [G, Wn]
    # [B, G, Wn, Hh, d] -> [B, Hh, G, Wn, d]
    qw = q[:, idx].transpose(0, 3, 1, 2, 4)
    kw = k[:, idx].transpose(0, 3, 1, 2, 4)
    vw = v[:, idx].transpose(0, 3, 1, 2, 4)
    ow = softmax_attention(qw, kw, vw, s)               # [B, Hh, G, Wn, d]
    o = np.empty_like(v)
    o[:, idx] = ow.transpose(0, 2, 3, 1, 4)
    return o


def global_pass(q, k, v, grid, tile, scale=None) -> np.ndarray:
    """Attn_G: softmax attention among the tokens sharing one offset, across windows.

    gist.science technical summary, "1. SQuad-Attention Operator", Global Pass.
    Here v is the value stream, which in the operator is the local pass's output.
    """
    q, k, v = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v")))
    s = _default_scale(q.shape[-1], scale)
    if not is_whole(grid, tile):
        return _unit_attention(q, k, v, padded_window_index(grid, tile).T, s)
    grp = window_index(grid, tile).T                    # [Wn, G]: group p = tokens at offset p
    qg = q[:, grp].transpose(0, 3, 1, 2, 4)             # [B, Hh, Wn, G, d]
    kg = k[:, grp].transpose(0, 3, 1, 2, 4)
    vg = v[:, grp].transpose(0, 3, 1, 2, 4)
    og = softmax_attention(qg, kg, vg, s)
    o = np.empty_like(v)
    o[:, grp] = og.transpose(0, 2, 3, 1, 4)
    return o


def _unit_attention(q, k, v, units, s) -> np.ndarray:
    """Softmax attention inside each unit (a row of `units`, -1 = absent token).

    Every token of the grid belongs to exactly one unit; each unit is attended
    on its own, over its present tokens only.
    """
    o = np.empty_like(v)
    for row in units:
        tok = row[row >= 0]
        qu = q[:, tok].transpose(0, 2, 1, 3)            # [B, Hh, L, d]
        ku = k[:, tok].transpose(0, 2, 1, 3)
        vu = v[:, tok].transpose(0, 2, 1, 3)
        o[:, tok] = softmax_attention(qu, ku, vu, s).transpose(0, 2, 1, 3)
    return o


def squad_forward(q, k, v, grid, tile, scale=None) -> np.ndarray:
    """SQuad-Attention forward: out = Attn_G(q, k, Attn_L(q, k, v)).

    The local output feeds the value stream of the global pass (gist.science
    technical summary, "1. SQuad-Attention Operator", Compositie).
    """
    o1 = local_pass(q, k, v, grid, tile, scale)
    return global_pass(q, k, o1, grid, tile, scale)


def squad_forward_groups(q, k, v, grid, tile, offsets, scale=None):
    """Rows of squad_forward for the chosen offset groups only.

    For offset p the global pass needs the local output only at the tokens of
    group p, and each of those is one query row of a local-pass window.  This
    computes exactly those rows, then the global pass over each chosen group; it
    is the same definition restricted to a subset of outputs, used to check
    full-size results by sampling.

    Returns (tokens [P, G] int64, out [B, P, G, Hh, d]) where tokens[i, g] is the
    token index of window g's member of group offsets[i].
    """
    q, k, v = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v")))
    idx = window_index(grid, tile)                      # [G, Wn]
    offsets = np.asarray(offsets, dtype=np.int64).reshape(-1)
    s = _default_scale(q.shape[-1], scale)
    kw = k[:, idx].transpose(0, 3, 1, 2, 4)             # [B, Hh, G, Wn, d]
    vw = v[:, idx].transpose(0, 3, 1, 2, 4)
    tokens = idx[:, offsets].T.copy()                   # [P, G]
    outs = []
    for i, p in enumerate(offsets):
        tok = tokens[i]                                 # [G]
        qp = q[:, tok].transpose(0, 2, 1, 3)            # [B, Hh, G, d]
        # local pass, one query row (the token at offset p) per window
        o1p = softmax_attention(qp[:, :, :, None, :], kw, vw, s)[:, :, :, 0, :]
        kp = k[:, tok].transpose(0, 2, 1, 3)
        outp = softmax_attention(qp, kp, o1p, s)        # [B, Hh, G, d]
        outs.append(outp.transpose(0, 2, 1, 3))         # [B, G, Hh, d]
    return tokens, np.stack(outs, axis=1)


def dense_attention(q, k, v, scale=None) -> np.ndarray:
    """Full softmax self-attention over all n tokens, per batch element and head.

    The quadratic operator the method replaces (abstract, all pages).
    [B, n, Hh, d] -> [B, n, Hh, d].
    """
    q, k, v = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v")))
    s = _default_scale(q.shape[-1], scale)
    o = softmax_attention(q.transpose(0, 2, 1, 3), k.transpose(0, 2, 1, 3),
                          v.transpose(0, 2, 1, 3), s)
    return o.transpose(0, 2, 1, 3)


# ---- the tensor reshapings the method is built from (gist.science technical
# summary, "Belangrijkste Bijdragen": standard tensor reshaping and standard
# attention blocks) ----

def tile_gather(x, grid, tile) -> np.ndarray:
    """Token order [B, n, Hh, d] -> window-major [B, Hh, G, Wn, d]."""
    x = np.asarray(x)
    idx = window_index(grid, tile)
    return x[:, idx].transpose(0, 3, 1, 2, 4).copy()


def tile_scatter(y, grid, tile) -> np.ndarray:
    """Inverse of tile_gather: [B, Hh, G, Wn, d] -> token order [B, n, Hh, d]."""
    y = np.asarray(y)
    idx = window_index(grid, tile)
    B, Hh, G, Wn, d = y.shape
    out = np.empty((B, G * Wn, Hh, d), dtype=y.dtype)
    out[:, idx] = y.transpose(0, 2, 3, 1, 4)
    return out


def window_to_group(y) -> np.ndarray:
    """Window-major [B, Hh, G, Wn, d] -> offset-group-major [B, Hh, Wn, G, d]."""
    return np.ascontiguousarray(np.asarray(y).transpose(0, 1, 3, 2, 4))


def window_attn(q, k, v, scale=None) -> np.ndarray:
    """Independent softmax attention per unit: [U, L, d] each -> [U, L, d]."""
    q = np.asarray(q, dtype=np.float64)
    s = _default_scale(q.shape[-1], scale)
    return softmax_attention(q, k, v, s)


# ---- gradients (the fine-tuning the pages run, flow-matching SFT and DMD2 in the
# technical summary's "Methodologie" and "Experimentele Resultaten", needs the
# operator's gradients; the pages give no formula, so these are the chain rule
# applied to the definitions above) ----

def softmax_attention_backward(q, k, v, dout, scale):
    """Gradients of softmax_attention with respect to q, k and v, in float64.

    With l = scale * q k^T, a = softmax over the key axis, o = a v and an upstream
    gradient dout:
      dv = a^T dout;  da = dout v^T;
      dl_ij = a_ij * (da_ij - sum_m a_im da_im)   (the softmax Jacobian; the sum
              equals <dout_i, o_i>);
      dq = scale * dl k;  dk = scale * dl^T q.
    Shapes as in softmax_attention; returns (dq, dk, dv).
    """
    q, k, v, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    logits = float(scale) * np.matmul(q, np.swapaxes(k, -1, -2))
    logits = logits - logits.max(axis=-1, keepdims=True)
    a = np.exp(logits)
    a = a / a.sum(axis=-1, keepdims=True)
    dv = np.matmul(np.swapaxes(a, -1, -2), dout)
    da = np.matmul(dout, np.swapaxes(v, -1, -2))
    dl = a * (da - (a * da).sum(axis=-1, keepdims=True))
    dq = float(scale) * np.matmul(dl, k)
    dk = float(scale) * np.matmul(np.swapaxes(dl, -1, -2), q)
    return dq, dk, dv


def _units_backward(q, k, v, dout, units, s):
    """softmax_attention_backward inside each unit (a row of `units`, -1 = absent)."""
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    if (units >= 0).all():
        # [B, U, L, Hh, d] -> [B, Hh, U, L, d]
        g = lambda x: x[:, units].transpose(0, 3, 1, 2, 4)
        gq, gk, gv = softmax_attention_backward(g(q), g(k), g(v), g(dout), s)
        for dst, src in ((dq, gq), (dk, gk), (dv, gv)):
            dst[:, units] = src.transpose(0, 2, 3, 1, 4)
        return dq, dk, dv
    for row in units:
        tok = row[row >= 0]
        g = lambda x: x[:, tok].transpose(0, 2, 1, 3)
        gq, gk, gv = softmax_attention_backward(g(q), g(k), g(v), g(dout), s)
        for dst, src in ((dq, gq), (dk, gk), (dv, gv)):
            dst[:, tok] = src.transpose(0, 2, 1, 3)
    return dq, dk, dv


def local_pass_backward(q, k, v, dout, grid, tile, scale=None):
    """Gradients of local_pass (Attn_L) with respect to q, k, v; token order."""
    q, k, v, dout = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")))
    s = _default_scale(q.shape[-1], scale)
    return _units_backward(q, k, v, dout, padded_window_index(grid, tile), s)


def global_pass_backward(q, k, v, dout, grid, tile, scale=None):
    """Gradients of global_pass (Attn_G, value stream v) with respect to q, k, v."""
    q, k, v, dout = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")))
    s = _default_scale(q.shape[-1], scale)
    return _units_backward(q, k, v, dout, padded_window_index(grid, tile).T.copy(), s)


def squad_backward(q, k, v, dout, grid, tile, scale=None):
    """Gradients of squad_forward with respect to q, k and v, given dout.

    out = Attn_G(q, k, o1) with o1 = Attn_L(q, k, v).  q and k enter both passes,
    so their gradients are the sums of the two passes' gradients; the global
    pass's value gradient is the upstream gradient of the local output:
      (dq_G, dk_G, do1) = Attn_G backward at (q, k, o1, dout)
      (dq_L, dk_L, dv)  = Attn_L backward at (q, k, v, do1)
      dq = dq_G + dq_L,  dk = dk_G + dk_L.
    """
    o1 = local_pass(q, k, v, grid, tile, scale)
    dq_g, dk_g, do1 = global_pass_backward(q, k, o1, dout, grid, tile, scale)
    dq_l, dk_l, dv = local_pass_backward(q, k, v, do1, grid, tile, scale)
    return dq_g + dq_l, dk_g + dk_l, dv


def squad_forward_stats(q, k, grid, tile, scale=None):
    """Per-row softmax statistics of both passes: the natural-log normaliser
    lse_i = log sum_j exp(scale * <q_i, k_j>) over row i's unit, for the local pass
    (unit = window) and the global pass (unit = offset group).  Token order
    [B, n, Hh] each; returns (lse_local, lse_global)."""
    q = _as_bnhd(q, "q")
    k = _as_bnhd(k, "k")
    s = _default_scale(q.shape[-1], scale)
    out = []
    for units in (padded_window_index(grid, tile), padded_window_index(grid, tile).T):
        lse = np.zeros(q.shape[:3])
        for row in units:
            tok = row[row >= 0]
            qu = q[:, tok].transpose(0, 2, 1, 3)        # [B, Hh, L, d]
            ku = k[:, tok].transpose(0, 2, 1, 3)
            l = s * np.matmul(qu, np.swapaxes(ku, -1, -2))
            m = l.max(axis=-1, keepdims=True)
            lse[:, tok] = (m[..., 0] + np.log(np.exp(l - m).sum(axis=-1))).transpose(0, 2, 1)
        out.append(lse)
    return tuple(out)


# ---- more than two passes (the pages name composing more than two passes as
# future work, to trade depth for efficiency; technical summary, "Betekenis en
# Claims") ----

def _kpass_levels(grid, tiles):
    """Per-axis level sizes of a nested tiling: tiles[0] | tiles[1] | ... | grid."""
    T, H, W = (int(x) for x in grid)
    ext = [(1, 1, 1)] + [tuple(int(x) for x in t) for t in tiles] + [(T, H, W)]
    for a, b in zip(ext[:-1], ext[1:]):
        for x, y in zip(a, b):
            if x <= 0 or y % x:
                raise ValueError(f"tiles {tiles} are not nested in grid {grid}")
    return ext


def kpass_level_index(grid, tiles, level):
    """Units of pass `level` (0-based) of the k-pass operator: int64 idx[U, L].

    With nested tiles t1 | t2 | ... | t(k-1) | grid, a token's coordinate on each
    axis splits into k digits: digit j is its position among the t(j)-tiles inside
    its t(j+1)-tile (t0 = 1 cell, tk = the grid).  Pass j mixes the tokens that
    agree on every digit except digit j: row r of idx lists the L tokens of one
    unit, ordered by their level-j digits row-major over (t, h, w); units run over
    the other digits.  k = 2 gives the local pass (level 0, units = windows) and
    the global pass (level 1, units = offsets).
    """
    ext = _kpass_levels(grid, tiles)
    T, H, W = (int(x) for x in grid)
    k = len(ext) - 1
    coords = np.stack(np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij"), -1).reshape(-1, 3)
    tok = (coords[:, 0] * H + coords[:, 1]) * W + coords[:, 2]
    # digit j on axis a: (x // ext[j][a]) % (ext[j+1][a] // ext[j][a])
    digits = [np.stack([(coords[:, a] // ext[j][a]) % (ext[j + 1][a] // ext[j][a]) for a in range(3)], -1)
              for j in range(k)]
    radix = [tuple(ext[j + 1][a] // ext[j][a] for a in range(3)) for j in range(k)]
    row = (digits[level][:, 0] * radix[level][1] + digits[level][:, 1]) * radix[level][2] + digits[level][:, 2]
    unit = np.zeros(len(tok), dtype=np.int64)
    for j in range(k):
        if j == level:
            continue
        d = digits[j]
        unit = ((unit * radix[j][0] + d[:, 0]) * radix[j][1] + d[:, 1]) * radix[j][2] + d[:, 2]
    L = int(np.prod(radix[level]))
    idx = np.empty((len(tok) // L, L), dtype=np.int64)
    idx[unit, row] = tok
    return idx


def squad_kpass_forward(q, k, v, grid, tiles, scale=None):
    """The operator with k = len(tiles) + 1 composed passes: o_0 = v and
    o_(j+1) = pass j (q, k, o_j), each pass the standard softmax attention inside
    its units (kpass_level_index); the output is o_k.  Same q and k in every pass,
    as in the two-pass operator, of which this is the k-level form (k = 2: tiles =
    [tile])."""
    q, k, v = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v")))
    s = _default_scale(q.shape[-1], scale)
    o = v
    for level in range(len(tiles) + 1):
        idx = kpass_level_index(grid, tiles, level)
        g = lambda x: x[:, idx].transpose(0, 3, 1, 2, 4)    # [B, Hh, U, L, d]
        ou = softmax_attention(g(q), g(k), g(o), s)
        o = np.empty_like(v)
        o[:, idx] = ou.transpose(0, 2, 3, 1, 4)
    return o


def squad_kpass_backward(q, k, v, dout, grid, tiles, scale=None):
    """Gradients of squad_kpass_forward with respect to q, k and v, given dout.

    The chain rule over the levels, from the last down: with o_0 = v and
    o_(j+1) = Attn_j(q, k, o_j), the upstream gradient of o_k is dout, and level j's
    backward at (q, k, o_j) given the gradient of o_(j+1) yields its parts of dq and
    dk and the gradient of o_j; dq and dk are the sums over the levels, dv is the
    gradient of o_0.  Two levels give squad_backward.
    """
    q, k, v, dout = (_as_bnhd(x, nm) for x, nm in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")))
    s = _default_scale(q.shape[-1], scale)
    levels = len(tiles) + 1
    outs = [v]
    for level in range(levels - 1):
        idx = kpass_level_index(grid, tiles, level)
        g = lambda x: x[:, idx].transpose(0, 3, 1, 2, 4)
        ou = softmax_attention(g(q), g(k), g(outs[-1]), s)
        o = np.empty_like(v)
        o[:, idx] = ou.transpose(0, 2, 3, 1, 4)
        outs.append(o)
    dq, dk = np.zeros_like(q), np.zeros_like(k)
    grad = np.asarray(dout, np.float64)
    for level in reversed(range(levels)):
        gq, gk, grad = _units_backward(q, k, outs[level], grad, kpass_level_index(grid, tiles, level), s)
        dq += gq
        dk += gk
    return dq, dk, grad


# ---- the attention block around the operator (the pages time attention per block
# of a 5B video DiT; technical summary, "Experimentele Resultaten") ----

def squad_block_forward(x, w_qkv, w_out, grid, tile, heads, scale=None, dense=False):
    """y = Attn(q, k, v) w_out^T with [q | k | v] = x w_qkv^T, in float64.

    x [B, n, hidden]; w_qkv [3 hidden, hidden] and w_out [hidden, hidden] in the
    nn.Linear layout (out_features, in_features); q, k, v are the three column
    blocks of the projection, each split into `heads` heads of hidden / heads.
    Attn is squad_forward (dense=True: dense_attention, the comparator).  No bias
    and no normalisation: the pages describe neither.
    """
    x = np.asarray(x, dtype=np.float64)
    B, n, hidden = x.shape
    d = hidden // int(heads)
    qkv = np.matmul(x, np.asarray(w_qkv, np.float64).T)                  # [B, n, 3 hidden]
    q, k, v = (qkv[..., i * hidden:(i + 1) * hidden].reshape(B, n, heads, d) for i in range(3))
    a = dense_attention(q, k, v, scale) if dense else squad_forward(q, k, v, grid, tile, scale)
    return np.matmul(a.reshape(B, n, hidden), np.asarray(w_out, np.float64).T)
