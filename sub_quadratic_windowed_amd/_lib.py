"""ctypes view of libsquad.so (the C ABI declared in include/squad.h)."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# SQUAD_LIBRARY may point at another build of the same C ABI (for A/B comparisons)
LIB_PATH = os.environ.get("SQUAD_LIBRARY") or os.path.join(_HERE, "libsquad.so")

STATUS_NAMES = {
    0: "SQUAD_OK",
    1: "SQUAD_ERR_INVALID_ARG",
    2: "SQUAD_ERR_SHAPE",
    3: "SQUAD_ERR_UNSUPPORTED",
    4: "SQUAD_ERR_ALIAS",
    5: "SQUAD_ERR_ALIGN",
    6: "SQUAD_ERR_WORKSPACE",
    7: "SQUAD_ERR_HIP",
    8: "SQUAD_ERR_SCRATCH",
}

# bytes of device scratch squad_attn_forward_noalloc holds per device
# (SQUAD_NOALLOC_SCRATCH_BYTES in include/squad.h)
NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = [
    "squad_status_string",
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
    "squad_kpass_workspace_size",
    "squad_kpass_forward",
    "squad_debug_kpass_offsets",
    "squad_block_workspace_size",
    "squad_block_forward",
    "squad_debug_mfma_probe",
    "squad_kpass_train_workspace_size",
    "squad_kpass_forward_train",
    "squad_kpass_backward",
    "squad_attn_forward_noalloc",
    "squad_blas_create",
    "squad_blas_destroy",
]

_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
I3 = ctypes.POINTER(ctypes.c_int32)
F = ctypes.c_float
SZ = ctypes.c_size_t


def _declare(lib):
    lib.squad_status_string.argtypes = [ctypes.c_int]
    lib.squad_status_string.restype = ctypes.c_char_p
    lib.squad_attn_forward.argtypes = [P, P, P, I3, I3, I32, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_attn_forward.restype = ctypes.c_int
    lib.squad_attn_forward_noalloc.argtypes = [P, P, P, I3, I3, I32, P, I32, I32, I32, F, P]
    lib.squad_attn_forward_noalloc.restype = ctypes.c_int
    lib.squad_attn_forward_local.argtypes = [P, P, P, I3, I3, I32, I32, I32, I32, F, P, SZ, P]
    lib.squad_attn_forward_local.restype = ctypes.c_int
    lib.squad_attn_forward_global.argtypes = [P, P, I3, I3, I32, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_attn_forward_global.restype = ctypes.c_int
    lib.squad_attn_workspace_size.argtypes = [I3, I3, I32, I32, I32, I32]
    lib.squad_attn_workspace_size.restype = SZ
    lib.squad_attn_train_workspace_size.argtypes = [I3, I3, I32, I32, I32, I32]
    lib.squad_attn_train_workspace_size.restype = SZ
    lib.squad_attn_forward_train.argtypes = [P, P, P, I3, I3, I32, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_attn_forward_train.restype = ctypes.c_int
    lib.squad_attn_backward.argtypes = [P, P, P, P, P, I3, I3, I32, P, P, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_attn_backward.restype = ctypes.c_int
    lib.squad_kpass_workspace_size.argtypes = [I3, I3, I32, I32, I32, I32, I32]
    lib.squad_kpass_workspace_size.restype = SZ
    lib.squad_kpass_forward.argtypes = [P, P, P, I3, I3, I32, I32, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_kpass_forward.restype = ctypes.c_int
    lib.squad_debug_kpass_offsets.argtypes = [I3, I3, I32, I32, I32, I32, I32, ctypes.POINTER(ctypes.c_int64)]
    lib.squad_debug_kpass_offsets.restype = ctypes.c_int
    lib.squad_block_workspace_size.argtypes = [I3, I3, I32, I32, I32, I32]
    lib.squad_block_workspace_size.restype = SZ
    lib.squad_block_forward.argtypes = [P, P, P, I3, I3, I32, P, I32, I32, I32, F, I32, P, P, SZ, P]
    lib.squad_blas_create.argtypes = [ctypes.POINTER(P)]
    lib.squad_blas_create.restype = ctypes.c_int
    lib.squad_blas_destroy.argtypes = [P]
    lib.squad_blas_destroy.restype = ctypes.c_int
    lib.squad_block_forward.restype = ctypes.c_int
    lib.squad_debug_mfma_probe.argtypes = [P, I32, I32, P]
    lib.squad_debug_mfma_probe.restype = ctypes.c_int
    lib.squad_kpass_train_workspace_size.argtypes = [I3, I3, I32, I32, I32, I32, I32]
    lib.squad_kpass_train_workspace_size.restype = SZ
    lib.squad_kpass_forward_train.argtypes = [P, P, P, I3, I3, I32, I32, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_kpass_forward_train.restype = ctypes.c_int
    lib.squad_kpass_backward.argtypes = [P, P, P, P, P, I3, I3, I32, I32, P, P, P, I32, I32, I32, F, P, SZ, P]
    lib.squad_kpass_backward.restype = ctypes.c_int
    lib.squad_plan_tile.argtypes = [I3, I3]
    lib.squad_plan_tile.restype = ctypes.c_int
    for name in ("squad_local_pass", "squad_global_pass"):
        f = getattr(lib, name)
        f.argtypes = [P, P, P, I3, I3, I32, P, I32, I32, I32, F, P]
        f.restype = ctypes.c_int
    for name in ("squad_tile_gather", "squad_tile_scatter", "squad_window_to_group"):
        f = getattr(lib, name)
        f.argtypes = [P, P, I3, I3, I32, I32, I32, I32, P]
        f.restype = ctypes.c_int
    lib.squad_window_attn.argtypes = [P, P, P, P, I32, I32, I32, I32, F, P]
    lib.squad_window_attn.restype = ctypes.c_int
    lib.squad_dense_attn_forward.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, F, P]
    lib.squad_dense_attn_forward.restype = ctypes.c_int
    lib.squad_debug_row_offsets.argtypes = [I32, I3, I3, I32, I32, I32, ctypes.POINTER(ctypes.c_int64)]
    lib.squad_debug_row_offsets.restype = ctypes.c_int


def lib():
    """The loaded library; raises if libsquad.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m sub_quadratic_windowed_amd.build` "
                "(there is no fallback implementation)")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


def int3(x):
    vals = [int(v) for v in x]
    if len(vals) != 3:
        raise ValueError(f"expected three sizes, got {x!r}")
    return (ctypes.c_int32 * 3)(*vals)
