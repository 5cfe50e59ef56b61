"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  There is no fallback of any kind; if the library is missing the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1

MOE_ACT_GELU = 0
MOE_ACT_SILU = 1

MOE_OK = 0
MOE_ERR_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_ERR_SCRATCH = 5

# bytes of the fixed device scratch of moe_forward_noalloc
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 8
MOE_MAX_SHARED = 8
MOE_NUM_STAGE_EVENTS = 7

# names of the C ABI entry points (include/moe.h)
EXPORTS = ("moe_forward", "moe_workspace_bytes", "moe_status_string", "moe_forward_expert_choice",
           "moe_workspace_bytes_expert_choice", "moe_quantize_mxfp8", "moe_workspace_bytes_mxfp8",
           "moe_forward_mxfp8", "moe_expert_choice_capacity", "moe_forward_noalloc", "moe_pack_weights")


class MoeLaunch(ctypes.Structure):
    """Mirror of moe_launch_t."""
    _fields_ = [
        ("T", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("h", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("b_g", ctypes.c_void_p),
        ("expert_counts", ctypes.c_void_p),
        ("expert_kept", ctypes.c_void_p),
        ("slot_pos", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("stage_events", ctypes.c_void_p),
        ("z_loss", ctypes.c_void_p),
        ("activation", ctypes.c_int32),
        ("min_capacity", ctypes.c_int32),
        ("b_sel", ctypes.c_void_p),
        ("weights_packed", ctypes.c_int32),
    ]


def _load():
    # torch ships its own HIP runtime.  Loading torch first puts that runtime in
    # the process's global symbol scope, so libmoe's HIP calls bind to it and the
    # process has one runtime: torch's device pointers and streams are then valid
    # in libmoe's launches.  Loaded the other way round, libmoe would bind to a
    # second runtime that cannot open the device while torch's holds it.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_mixture_experts_28_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.moe_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_workspace_bytes.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_int]
    lib.moe_workspace_bytes_expert_choice.restype = ctypes.c_size_t
    lib.moe_workspace_bytes_expert_choice.argtypes = [ctypes.c_int32] * 6 + [ctypes.c_int]
    lib.moe_forward_expert_choice.restype = ctypes.c_int
    lib.moe_forward_expert_choice.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(MoeLaunch),
    ]
    lib.moe_quantize_mxfp8.restype = ctypes.c_int
    lib.moe_quantize_mxfp8.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_workspace_bytes_mxfp8.restype = ctypes.c_size_t
    lib.moe_workspace_bytes_mxfp8.argtypes = [ctypes.c_int32] * 6
    lib.moe_forward_mxfp8.restype = ctypes.c_int
    lib.moe_forward_mxfp8.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(MoeLaunch),
    ]
    lib.moe_pack_weights.restype = ctypes.c_int
    lib.moe_pack_weights.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_expert_choice_capacity.restype = ctypes.c_int32
    lib.moe_expert_choice_capacity.argtypes = [ctypes.c_float, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_forward_noalloc.restype = ctypes.c_int
    lib.moe_forward_noalloc.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(MoeLaunch),
    ]
    lib.moe_forward.restype = ctypes.c_int
    lib.moe_forward.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.POINTER(MoeLaunch),
    ]
    return lib


LIB = _load()


def moe_workspace_bytes(T: int, d: int, h: int, E: int, k: int, n_shared: int, dtype: int) -> int:
    return int(LIB.moe_workspace_bytes(T, d, h, E, k, n_shared, dtype))


def moe_workspace_bytes_expert_choice(T: int, d: int, h: int, E: int, C: int, n_shared: int, dtype: int) -> int:
    return int(LIB.moe_workspace_bytes_expert_choice(T, d, h, E, C, n_shared, dtype))


def moe_expert_choice_capacity(capacity_factor: float, T: int, E: int, min_capacity: int = 0) -> int:
    """Raw call: tokens per expert under expert choice, or -1 for invalid arguments."""
    return int(LIB.moe_expert_choice_capacity(capacity_factor, T, E, min_capacity))


def moe_status_string(status: int) -> str:
    return LIB.moe_status_string(status).decode()


def moe_forward(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w, aux_loss,
                launch: MoeLaunch) -> int:
    """Raw call of the C entry point: every array argument is a device address (int)."""
    return int(LIB.moe_forward(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w,
                               aux_loss, ctypes.byref(launch)))


def moe_forward_noalloc(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w, aux_loss,
                        launch: MoeLaunch) -> int:
    """Raw call of the entry point that takes no workspace (the library's fixed
    device scratch; launch.workspace is ignored)."""
    return int(LIB.moe_forward_noalloc(x, W_g, W1, b1, W2, b2, E, k, capacity_factor, n_shared, out, topk_idx,
                                       topk_w, aux_loss, ctypes.byref(launch)))


def moe_forward_expert_choice(x, W_g, W1, b1, W2, b2, E, C, n_shared, out, ec_token, ec_w, aux_loss,
                              launch: MoeLaunch) -> int:
    """Raw call of the expert-choice entry point: every array argument is a device address (int)."""
    return int(LIB.moe_forward_expert_choice(x, W_g, W1, b1, W2, b2, E, C, n_shared, out, ec_token, ec_w,
                                             aux_loss, ctypes.byref(launch)))


def moe_pack_weights(W, n_mat: int, N: int, K: int, dtype: int, Wp, stream) -> int:
    """moe_pack_weights: W [n_mat, N, K] bf16 -> the tile-packed layout in Wp."""
    return int(LIB.moe_pack_weights(W, n_mat, N, K, dtype, Wp, stream))


def moe_quantize_mxfp8(src, rows: int, cols: int, codes, scales, stream) -> int:
    """Raw call: bf16 [rows, cols] at device address src -> MXFP8 codes / scales."""
    return int(LIB.moe_quantize_mxfp8(src, rows, cols, codes, scales, stream))


def moe_workspace_bytes_mxfp8(T: int, d: int, h: int, E: int, k: int, n_shared: int) -> int:
    return int(LIB.moe_workspace_bytes_mxfp8(T, d, h, E, k, n_shared))


def moe_forward_mxfp8(x, W_g, W1, W1s, b1, W2, W2s, b2, E, k, capacity_factor, n_shared, out, topk_idx, topk_w,
                      aux_loss, launch: MoeLaunch) -> int:
    """Raw call of the MXFP8 entry point: every array argument is a device address (int)."""
    return int(LIB.moe_forward_mxfp8(x, W_g, W1, W1s, b1, W2, W2s, b2, E, k, capacity_factor, n_shared, out,
                                     topk_idx, topk_w, aux_loss, ctypes.byref(launch)))
