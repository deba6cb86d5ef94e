"""SQuad-Attention forward on AMD MI355X: thin Python binding over libsquad.so.

Every function here only checks and marshals arguments and calls the C ABI of the
same name (include/squad.h); all arithmetic runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  There is no fallback: if
the library is missing, calls raise.

Token-order tensors are [batch, n, heads, head_dim] with n = T*H*W tokens of a
T x H x W latent grid numbered row-major over (t, h, w); a window is a
tt x th x tw tile of that grid.
"""

import ctypes

import torch

from . import _lib

__all__ = [
    "SquadError",
    "squad_attn_forward",
    "squad_attn_workspace_size",
    "squad_plan_tile",
    "squad_attn_forward_local",
    "squad_attn_forward_global",
    "squad_local_pass",
    "squad_global_pass",
    "squad_tile_gather",
    "squad_tile_scatter",
    "squad_window_to_group",
    "squad_window_attn",
    "squad_dense_attn_forward",
    "squad_debug_row_offsets",
    "squad_attn_train_workspace_size",
    "squad_attn_forward_train",
    "squad_attn_backward",
    "SquadAttention",
    "squad_kpass_workspace_size",
    "squad_kpass_forward",
    "squad_debug_kpass_offsets",
    "squad_debug_mfma_probe",
    "squad_kpass_train_workspace_size",
    "squad_kpass_forward_train",
    "squad_kpass_backward",
    "squad_block_workspace_size",
    "squad_block_forward",
    "BlasHandle",
    "squad_attn_forward_noalloc",
    "DTYPE_CODES",
]

DTYPE_CODES = {torch.float32: 0, torch.bfloat16: 1}


class SquadError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.lib().squad_status_string(status).decode()
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)}: {msg}")


def _check(status, where):
    if status != 0:
        raise SquadError(status, where)


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _tensor(x, name, ndim=None, dtype=None, device=None):
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {x.device})")
    if x.dtype not in DTYPE_CODES:
        raise ValueError(f"{name} must be float32 or bfloat16 (got {x.dtype})")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name} has dtype {x.dtype}, expected {dtype}")
    if device is not None and x.device != device:
        raise ValueError(f"{name} is on {x.device}, expected {device}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and x.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(x.shape)}")
    return x


def _ptr(x):
    return ctypes.c_void_p(x.data_ptr())


def _scale(scale):
    return ctypes.c_float(0.0 if scale is None else float(scale))


def _token_inputs(q, k, v, grid, heads):
    q = _tensor(q, "q", 4)
    k = _tensor(k, "k", 4, q.dtype, q.device)
    v = _tensor(v, "v", 4, q.dtype, q.device)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    B, n, Hh, d = q.shape
    if heads is not None and int(heads) != Hh:
        raise ValueError(f"heads={heads} but q has {Hh} heads")
    T, H, W = (int(x) for x in grid)
    if T * H * W != n:
        raise ValueError(f"grid {tuple(grid)} has {T * H * W} tokens, q has {n}")
    return q, k, v, B, n, Hh, d


def _out_like(out, q, name="out"):
    if out is None:
        return torch.empty_like(q)
    out = _tensor(out, name, 4, q.dtype, q.device)
    if out.shape != q.shape:
        raise ValueError(f"{name} shape {tuple(out.shape)} != {tuple(q.shape)}")
    return out


def squad_attn_workspace_size(grid, tile, heads, batch, head_dim, dtype):
    """Bytes of workspace squad_attn_forward needs (0 for invalid arguments)."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().squad_attn_workspace_size(_lib.int3(grid), _lib.int3(tile), int(heads),
                                                    int(batch), int(head_dim), code))


def squad_plan_tile(grid):
    """The tile (tt, th, tw) the library's planner picks for a T x H x W grid: the
    least product work over whole and cut tilings (host-only, no device needed)."""
    out = (ctypes.c_int32 * 3)()
    _check(_lib.lib().squad_plan_tile(_lib.int3(grid), out), "squad_plan_tile")
    return tuple(int(x) for x in out)


def squad_attn_forward(q, k, v, grid, tile, heads=None, out=None, scale=None, workspace=None,
                       stream=None):
    """SQuad-Attention forward: local windowed pass, then the global same-offset pass
    with the local output as value stream.  Returns out [batch, n, heads, head_dim]."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q)
    workspace = _workspace(workspace, squad_attn_workspace_size(grid, tile, Hh, B, d, q.dtype), q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.lib().squad_attn_forward(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), _lib.int3(tile), Hh, _ptr(out), B, d,
        DTYPE_CODES[q.dtype], _scale(scale), _ptr(workspace), ws_bytes, _stream(stream, q.device))
    _check(st, "squad_attn_forward")
    return out


def squad_attn_forward_noalloc(q, k, v, grid, tile, heads=None, out=None, scale=None, stream=None):
    """squad_attn_forward without a workspace: the library keeps the local output in
    its own per-device scratch array (for callers that cannot allocate, such as
    code under graph capture).  Pass `out` to make the call allocate nothing at
    all; calls that overlap in time on one device must not be issued."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q)
    st = _lib.lib().squad_attn_forward_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), _lib.int3(tile), Hh, _ptr(out), B, d,
        DTYPE_CODES[q.dtype], _scale(scale), _stream(stream, q.device))
    _check(st, "squad_attn_forward_noalloc")
    return out


def _workspace(workspace, need, device):
    if workspace is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace


def squad_attn_train_workspace_size(grid, tile, heads, batch, head_dim, dtype):
    """Bytes of the workspace squad_attn_forward_train and squad_attn_backward share."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().squad_attn_train_workspace_size(_lib.int3(grid), _lib.int3(tile), int(heads),
                                                          int(batch), int(head_dim), code))


def squad_attn_forward_train(q, k, v, grid, tile, heads=None, out=None, scale=None, workspace=None,
                             stream=None):
    """squad_attn_forward that also keeps what the backward needs in the workspace.
    Returns (out, workspace)."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q)
    workspace = _workspace(workspace, squad_attn_train_workspace_size(grid, tile, Hh, B, d, q.dtype), q.device)
    st = _lib.lib().squad_attn_forward_train(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), _lib.int3(tile), Hh, _ptr(out), B, d,
        DTYPE_CODES[q.dtype], _scale(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device))
    _check(st, "squad_attn_forward_train")
    return out, workspace


def squad_attn_backward(q, k, v, out, dout, grid, tile, workspace, heads=None, dq=None, dk=None, dv=None,
                        scale=None, stream=None):
    """Gradients (dq, dk, dv) of squad_attn_forward given dout; `workspace` as left by
    squad_attn_forward_train on the same inputs."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _tensor(out, "out", 4, q.dtype, q.device)
    dout = _tensor(dout, "dout", 4, q.dtype, q.device)
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    dq, dk, dv = (_out_like(x, q, nm) for x, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    workspace = _workspace(workspace, 0, q.device)
    st = _lib.lib().squad_attn_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _lib.int3(grid), _lib.int3(tile), Hh,
        _ptr(dq), _ptr(dk), _ptr(dv), B, d, DTYPE_CODES[q.dtype], _scale(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_attn_backward")
    return dq, dk, dv


class SquadAttention(torch.autograd.Function):
    """Autograd wrapper: out = SquadAttention.apply(q, k, v, grid, tile[, scale]).
    The forward keeps the library's training workspace; the backward calls
    squad_attn_backward (no arithmetic in Python)."""

    @staticmethod
    def forward(ctx, q, k, v, grid, tile, scale=None):
        q, k, v = (x.contiguous() for x in (q, k, v))
        out, ws = squad_attn_forward_train(q, k, v, tuple(grid), tuple(tile), scale=scale)
        ctx.save_for_backward(q, k, v, out, ws)
        ctx.geom = (tuple(grid), tuple(tile), scale)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, ws = ctx.saved_tensors
        grid, tile, scale = ctx.geom
        dq, dk, dv = squad_attn_backward(q, k, v, out, dout.contiguous(), grid, tile, ws, scale=scale)
        return dq, dk, dv, None, None, None


def _tiles(tiles):
    flat = [int(x) for t in tiles for x in t]
    if len(flat) != 3 * len(tiles) or not tiles:
        raise ValueError("tiles must be a non-empty list of (tt, th, tw)")
    return (ctypes.c_int32 * len(flat))(*flat), len(tiles) + 1


def squad_kpass_workspace_size(grid, tiles, heads, batch, head_dim, dtype):
    """Bytes of workspace squad_kpass_forward needs (0 for invalid arguments)."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    arr, levels = _tiles(tiles)
    return int(_lib.lib().squad_kpass_workspace_size(_lib.int3(grid), arr, levels, int(heads), int(batch),
                                                     int(head_dim), code))


def squad_kpass_forward(q, k, v, grid, tiles, heads=None, out=None, scale=None, workspace=None, stream=None):
    """The operator with len(tiles) + 1 composed passes over nested tiles
    tiles[0] | tiles[1] | ... | grid (include/squad.h); len(tiles) == 1 is
    squad_attn_forward with tile = tiles[0]."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q)
    arr, levels = _tiles(tiles)
    workspace = _workspace(workspace, squad_kpass_workspace_size(grid, tiles, Hh, B, d, q.dtype), q.device)
    st = _lib.lib().squad_kpass_forward(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), arr, levels, Hh, _ptr(out), B, d, DTYPE_CODES[q.dtype],
        _scale(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_kpass_forward")
    return out


def squad_block_workspace_size(grid, tile, heads, batch, head_dim, dtype):
    """Bytes of workspace squad_block_forward needs (0 for invalid arguments)."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(_lib.lib().squad_block_workspace_size(_lib.int3(grid), _lib.int3(tile), int(heads), int(batch),
                                                     int(head_dim), code))


class BlasHandle:
    """A rocBLAS handle from squad_blas_create for squad_block_forward, created on
    the current device and released with squad_blas_destroy when closed or
    collected."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check(_lib.lib().squad_blas_create(ctypes.byref(h)), "squad_blas_create")
        self.ptr = h

    def close(self):
        if self.ptr is not None and self.ptr.value:
            _lib.lib().squad_blas_destroy(self.ptr)
        self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_blas_handles = {}


def _blas_for(device):
    """The binding's own handle for `device` (one per device, kept by this module)."""
    key = device.index if device.index is not None else torch.cuda.current_device()
    if key not in _blas_handles:
        with torch.cuda.device(key):
            _blas_handles[key] = BlasHandle()
    return _blas_handles[key]


def squad_block_forward(x, w_qkv, w_out, grid, tile, heads, y=None, scale=None, dense=False, workspace=None,
                        stream=None, blas=None):
    """The attention block: y = SQuad(x w_qkv^T split into q, k, v) w_out^T (dense=True:
    full attention instead).  x [batch, n, hidden], w_qkv [3 hidden, hidden], w_out
    [hidden, hidden]; returns y [batch, n, hidden].  `blas`: a BlasHandle (by default
    the binding's own handle for x's device)."""
    x = _tensor(x, "x", 3)
    B, n, hidden = x.shape
    Hh = int(heads)
    if hidden % Hh:
        raise ValueError(f"hidden {hidden} is not a multiple of heads {Hh}")
    d = hidden // Hh
    w_qkv = _tensor(w_qkv, "w_qkv", 2, x.dtype, x.device)
    w_out = _tensor(w_out, "w_out", 2, x.dtype, x.device)
    if tuple(w_qkv.shape) != (3 * hidden, hidden) or tuple(w_out.shape) != (hidden, hidden):
        raise ValueError("w_qkv must be [3 hidden, hidden] and w_out [hidden, hidden]")
    T, H, W = (int(g) for g in grid)
    if T * H * W != n:
        raise ValueError(f"grid {tuple(grid)} has {T * H * W} tokens, x has {n}")
    if y is None:
        y = torch.empty_like(x)
    else:
        y = _tensor(y, "y", 3, x.dtype, x.device)
        if y.shape != x.shape:
            raise ValueError(f"y shape {tuple(y.shape)} != {tuple(x.shape)}")
    workspace = _workspace(workspace, squad_block_workspace_size(grid, tile, Hh, B, d, x.dtype), x.device)
    st = _lib.lib().squad_block_forward(
        _ptr(x), _ptr(w_qkv), _ptr(w_out), _lib.int3(grid), _lib.int3(tile), Hh, _ptr(y), B, d,
        DTYPE_CODES[x.dtype], _scale(scale), 1 if dense else 0, (blas or _blas_for(x.device)).ptr, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, x.device))
    _check(st, "squad_block_forward")
    return y


def squad_kpass_train_workspace_size(grid, tiles, heads, batch, head_dim, dtype):
    """Bytes of the workspace squad_kpass_forward_train and squad_kpass_backward share."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    arr, levels = _tiles(tiles)
    return int(_lib.lib().squad_kpass_train_workspace_size(_lib.int3(grid), arr, levels, int(heads), int(batch),
                                                           int(head_dim), code))


def squad_kpass_forward_train(q, k, v, grid, tiles, heads=None, out=None, scale=None, workspace=None,
                              stream=None):
    """squad_kpass_forward keeping what squad_kpass_backward needs.  Returns (out, workspace)."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q)
    arr, levels = _tiles(tiles)
    workspace = _workspace(workspace, squad_kpass_train_workspace_size(grid, tiles, Hh, B, d, q.dtype), q.device)
    st = _lib.lib().squad_kpass_forward_train(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), arr, levels, Hh, _ptr(out), B, d, DTYPE_CODES[q.dtype],
        _scale(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_kpass_forward_train")
    return out, workspace


def squad_kpass_backward(q, k, v, out, dout, grid, tiles, workspace, heads=None, dq=None, dk=None, dv=None,
                         scale=None, stream=None):
    """Gradients (dq, dk, dv) of squad_kpass_forward given dout; `workspace` as left by
    squad_kpass_forward_train on the same inputs."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _tensor(out, "out", 4, q.dtype, q.device)
    dout = _tensor(dout, "dout", 4, q.dtype, q.device)
    if out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("out and dout must have q's shape")
    dq, dk, dv = (_out_like(x, q, nm) for x, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")))
    arr, levels = _tiles(tiles)
    workspace = _workspace(workspace, 0, q.device)
    st = _lib.lib().squad_kpass_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _lib.int3(grid), arr, levels, Hh, _ptr(dq), _ptr(dk),
        _ptr(dv), B, d, DTYPE_CODES[q.dtype], _scale(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_kpass_backward")
    return dq, dk, dv


def squad_attn_forward_local(q, k, v, grid, tile, heads=None, scale=None, workspace=None, stream=None):
    """First half of squad_attn_forward: the local pass into the workspace (returned)."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    workspace = _workspace(workspace, squad_attn_workspace_size(grid, tile, Hh, B, d, q.dtype), q.device)
    st = _lib.lib().squad_attn_forward_local(
        _ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), _lib.int3(tile), Hh, B, d, DTYPE_CODES[q.dtype],
        _scale(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_attn_forward_local")
    return workspace


def squad_attn_forward_global(q, k, grid, tile, workspace, heads=None, out=None, scale=None, stream=None):
    """Second half of squad_attn_forward: the global pass over the workspace's local output."""
    q, k, _, B, n, Hh, d = _token_inputs(q, k, k, grid, heads)
    out = _out_like(out, q)
    workspace = _workspace(workspace, 0, q.device)
    st = _lib.lib().squad_attn_forward_global(
        _ptr(q), _ptr(k), _lib.int3(grid), _lib.int3(tile), Hh, _ptr(out), B, d, DTYPE_CODES[q.dtype],
        _scale(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    _check(st, "squad_attn_forward_global")
    return out


def squad_local_pass(q, k, v, grid, tile, heads=None, out=None, scale=None, stream=None):
    """Local pass alone: softmax attention inside each window (token order in and out)."""
    q, k, v, B, n, Hh, d = _token_inputs(q, k, v, grid, heads)
    out = _out_like(out, q, "o1")
    st = _lib.lib().squad_local_pass(_ptr(q), _ptr(k), _ptr(v), _lib.int3(grid), _lib.int3(tile), Hh,
                                     _ptr(out), B, d, DTYPE_CODES[q.dtype], _scale(scale),
                                     _stream(stream, q.device))
    _check(st, "squad_local_pass")
    return out


def squad_global_pass(q, k, vstream, grid, tile, heads=None, out=None, scale=None, stream=None):
    """Global pass alone: attention among same-offset tokens with `vstream` as values."""
    q, k, vstream, B, n, Hh, d = _token_inputs(q, k, vstream, grid, heads)
    out = _out_like(out, q)
    st = _lib.lib().squad_global_pass(_ptr(q), _ptr(k), _ptr(vstream), _lib.int3(grid), _lib.int3(tile),
                                      Hh, _ptr(out), B, d, DTYPE_CODES[q.dtype], _scale(scale),
                                      _stream(stream, q.device))
    _check(st, "squad_global_pass")
    return out


def _perm(fn_name, src, grid, tile, out_shape, dst, batch, heads, head_dim, stream):
    src = _tensor(src, "src")
    if dst is None:
        dst = torch.empty(out_shape, dtype=src.dtype, device=src.device)
    else:
        dst = _tensor(dst, "dst", None, src.dtype, src.device)
        if tuple(dst.shape) != tuple(out_shape):
            raise ValueError(f"dst shape {tuple(dst.shape)} != {tuple(out_shape)}")
    st = getattr(_lib.lib(), fn_name)(_ptr(src), _ptr(dst), _lib.int3(grid), _lib.int3(tile), heads,
                                      batch, head_dim, DTYPE_CODES[src.dtype], _stream(stream, src.device))
    _check(st, fn_name)
    return dst


def _geo(grid, tile):
    T, H, W = (int(x) for x in grid)
    tt, th, tw = (int(x) for x in tile)
    if min(tt, th, tw) <= 0 or T % tt or H % th or W % tw:
        return T * H * W, 0, 0
    Wn = tt * th * tw
    return T * H * W, (T * H * W) // Wn, Wn


def squad_tile_gather(src, grid, tile, dst=None, stream=None):
    """Token order [B, n, Hh, d] -> window-major [B, Hh, G, Wn, d] (exact copy)."""
    B, n, Hh, d = src.shape
    _, G, Wn = _geo(grid, tile)
    return _perm("squad_tile_gather", src, grid, tile, (B, Hh, G, Wn, d), dst, B, Hh, d, stream)


def squad_tile_scatter(src, grid, tile, dst=None, stream=None):
    """Window-major [B, Hh, G, Wn, d] -> token order [B, n, Hh, d] (exact copy)."""
    B, Hh, G, Wn, d = src.shape
    n, _, _ = _geo(grid, tile)
    return _perm("squad_tile_scatter", src, grid, tile, (B, n, Hh, d), dst, B, Hh, d, stream)


def squad_window_to_group(src, grid, tile, dst=None, stream=None):
    """Window-major [B, Hh, G, Wn, d] -> group-major [B, Hh, Wn, G, d] (exact copy)."""
    B, Hh, G, Wn, d = src.shape
    return _perm("squad_window_to_group", src, grid, tile, (B, Hh, Wn, G, d), dst, B, Hh, d, stream)


def squad_window_attn(q, k, v, out=None, scale=None, stream=None):
    """Independent softmax attention per unit: q, k, v [units, len, head_dim]."""
    q = _tensor(q, "q", 3)
    k = _tensor(k, "k", 3, q.dtype, q.device)
    v = _tensor(v, "v", 3, q.dtype, q.device)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    out = torch.empty_like(q) if out is None else _tensor(out, "out", 3, q.dtype, q.device)
    U, L, d = q.shape
    st = _lib.lib().squad_window_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(out), U, L, d, DTYPE_CODES[q.dtype],
                                      _scale(scale), _stream(stream, q.device))
    _check(st, "squad_window_attn")
    return out


def squad_dense_attn_forward(q, k, v, out=None, scale=None, stream=None):
    """Dense full softmax self-attention over all n tokens: [B, n, Hh, d] (comparator)."""
    q = _tensor(q, "q", 4)
    k = _tensor(k, "k", 4, q.dtype, q.device)
    v = _tensor(v, "v", 4, q.dtype, q.device)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    out = _out_like(out, q)
    B, n, Hh, d = q.shape
    st = _lib.lib().squad_dense_attn_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, n, Hh, d,
                                             DTYPE_CODES[q.dtype], _scale(scale), _stream(stream, q.device))
    _check(st, "squad_dense_attn_forward")
    return out


def squad_debug_mfma_probe(out, blocks, iters, stream=None):
    """Run the measuring kernel (blocks x 256 threads, `iters` rounds of four bf16
    MFMAs per wave) into `out` (float32, blocks * 256 entries on the GPU)."""
    out = _tensor(out, "out", 1, torch.float32)
    if out.numel() < int(blocks) * 256:
        raise ValueError("out must hold blocks * 256 floats")
    _check(_lib.lib().squad_debug_mfma_probe(_ptr(out), int(blocks), int(iters), _stream(stream, out.device)),
           "squad_debug_mfma_probe")
    return out


def squad_debug_kpass_offsets(grid, tiles, level, heads, batch, head_dim):
    """Host-side element offsets of pass `level`'s six-digit map; numpy int64."""
    import numpy as np

    arr, levels = _tiles(tiles)
    out = np.zeros(int(batch) * int(heads) * int(grid[0]) * int(grid[1]) * int(grid[2]), dtype=np.int64)
    st = _lib.lib().squad_debug_kpass_offsets(_lib.int3(grid), arr, levels, int(level), int(heads), int(batch),
                                              int(head_dim), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    _check(st, "squad_debug_kpass_offsets")
    return out


def squad_debug_row_offsets(which, grid, tile, heads, batch, head_dim):
    """Host-side element offsets the kernels use (see include/squad.h); numpy int64."""
    import numpy as np

    cells = 1   # G * Wn: tile cells of the (possibly cut) tiling, absent ones included
    for g, t in zip(grid, tile):
        cells *= -(-int(g) // int(t)) * int(t) if int(t) > 0 else 0
    out = np.zeros(int(batch) * int(heads) * max(cells, 1), dtype=np.int64)
    st = _lib.lib().squad_debug_row_offsets(int(which), _lib.int3(grid), _lib.int3(tile), int(heads),
                                            int(batch), int(head_dim),
                                            out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    _check(st, "squad_debug_row_offsets")
    return out
