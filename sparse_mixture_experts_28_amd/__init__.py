"""Sparse Mixture-of-Experts FFN layer forward on MI355X (gfx950).

The layer runs entirely in the HIP kernels of ``libmoe.so`` behind the C ABI
of ``include/moe.h``; this package binds that ABI with ctypes (the raw
``moe_forward`` / ``moe_workspace_bytes`` / ``moe_status_string``) and adds
``forward``, which only allocates the outputs and the workspace with torch and
passes torch's current stream.  Nothing here computes any part of the layer.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

from ._lib import (EXPORTS, LIB_PATH, MOE_ACT_GELU, MOE_ACT_SILU, MOE_BF16, MOE_ERR_ARG, MOE_ERR_HIP,
                   MOE_ERR_SCRATCH, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_F32, MOE_MAX_EXPERTS, MOE_MAX_SHARED,
                   MOE_MAX_TOPK, MOE_NOALLOC_SCRATCH_BYTES, MOE_NUM_STAGE_EVENTS, MOE_OK, MoeLaunch,
                   moe_expert_choice_capacity, moe_forward, moe_forward_expert_choice, moe_forward_noalloc,
                   moe_forward_mxfp8, moe_pack_weights, moe_quantize_mxfp8, moe_status_string, moe_workspace_bytes,
                   moe_workspace_bytes_expert_choice, moe_workspace_bytes_mxfp8)

ACTIVATIONS = {"gelu": MOE_ACT_GELU, "silu": MOE_ACT_SILU}

STAGES = ("router", "scan", "scatter", "expert_phase1", "expert_phase2", "combine")
# under expert choice the third stage is the per-expert selection
STAGES_EXPERT_CHOICE = ("router", "scan", "select", "expert_phase1", "expert_phase2", "combine")


@dataclass
class MoEOutput:
    out: "object"            # [T, d], dtype of x
    topk_idx: "object"       # [T, k] int32
    topk_w: "object"         # [T, k] float32
    aux_loss: "object"       # [1] float32
    z_loss: "object"         # [1] float32, router z-loss
    expert_counts: "object"  # [E] int32
    expert_kept: "object"    # [E] int32
    slot_pos: "object"       # [T, k] int32


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _check_tensors(x, W_g, W1, b1, W2, b2, b_g, n_shared: int, activation: str) -> None:
    """Shapes, dtypes and placement of the layer's inputs (b1, b2, b_g may be None)."""
    import torch
    dev = x.device
    for t in (x, W_g, W1, b1, W2, b2):
        if t is not None and (not t.is_cuda or t.device != dev or not t.is_contiguous() or t.dtype != x.dtype):
            raise ValueError("x, W_g, W1, b1, W2, b2 must be contiguous tensors of one dtype on one GPU")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    T, d = x.shape
    E = W_g.shape[0]
    h = W1.shape[1]
    S = n_shared
    if W_g.shape != (E, d) or W1.shape != (E + S, h, d) or W2.shape != (E + S, d, h) or \
            (b1 is not None and b1.shape != (E + S, h)) or (b2 is not None and b2.shape != (E + S, d)):
        raise ValueError("inconsistent shapes")
    if b_g is not None and (b_g.dtype != torch.float32 or b_g.shape != (E,) or b_g.device != dev
                            or not b_g.is_contiguous()):
        raise ValueError("b_g must be a contiguous float32 [E] on the same GPU")


def _check_b_sel(b_sel, E, dev):
    import torch
    if b_sel is not None and (b_sel.dtype != torch.float32 or b_sel.shape != (E,) or b_sel.device != dev
                              or not b_sel.is_contiguous()):
        raise ValueError("b_sel must be a contiguous float32 [E] on the same GPU")


def _launch(x, T, d, h, dt, b_g, workspace, zl, activation, min_capacity, stage_events, b_sel=None):
    """A moe_launch_t on torch's current stream; returns it and the event-handle
    array that must stay alive until the call returns."""
    import torch
    launch = MoeLaunch()
    launch.T, launch.d, launch.h, launch.dtype = T, d, h, dt
    launch.b_g = b_g.data_ptr() if b_g is not None else None
    launch.b_sel = b_sel.data_ptr() if b_sel is not None else None
    launch.workspace = workspace.data_ptr() if workspace is not None else None
    launch.workspace_bytes = workspace.numel() if workspace is not None else 0
    launch.stream = torch.cuda.current_stream(x.device).cuda_stream
    launch.z_loss = zl.data_ptr()
    launch.activation = ACTIVATIONS[activation]
    launch.min_capacity = int(min_capacity)
    ev_arr = None
    if stage_events is not None:
        if len(stage_events) != MOE_NUM_STAGE_EVENTS:
            raise ValueError(f"stage_events needs {MOE_NUM_STAGE_EVENTS} events")
        handles = [0 if e is None else int(e.cuda_event) for e in stage_events]
        if not all(h for h, e in zip(handles, stage_events) if e is not None):
            raise ValueError("record each stage event once before passing it (creates its handle)")
        ev_arr = (ctypes.c_void_p * MOE_NUM_STAGE_EVENTS)(*handles)
        launch.stage_events = ctypes.cast(ev_arr, ctypes.c_void_p)
    return launch, ev_arr


def forward(x, W_g, W1, b1, W2, b2, k: int, capacity_factor: float = 0.0, n_shared: int = 0, b_g=None,
            *, activation: str = "gelu", min_capacity: int = 0, stage_events: Optional[Sequence] = None,
            workspace=None, b_sel=None, noalloc: bool = False, weights_packed: bool = False) -> MoEOutput:
    """Run the layer on torch tensors that live on one GPU.

    x [T,d]; W_g [E,d]; W1 [E+S,h,d]; b1 [E+S,h] or None; W2 [E+S,d,h];
    b2 [E+S,d] or None (float32 or bfloat16, contiguous; None = bias-free
    Linear); b_g optional float32 [E] added to the logits; b_sel optional
    float32 [E] seen by the top-k choice only (moe_launch_t.b_sel).
    ``activation`` is "gelu" or "silu"; ``min_capacity`` floors the capacity
    when capacity_factor > 0.
    ``stage_events``: optional list of MOE_NUM_STAGE_EVENTS torch.cuda.Event
    objects (already recorded once, so their handles exist) or None entries
    (skipped) that the library records at its stage boundaries.  ``noalloc``: call moe_forward_noalloc,
    whose scratch is the library's fixed device array (no workspace is
    allocated; problems beyond its size raise).  ``weights_packed``: W1 and
    W2 are ``pack_weights`` outputs (same shapes and dtype; bf16, d and h
    multiples of 256).  Raises RuntimeError on a non-zero status.
    """
    import torch
    _check_tensors(x, W_g, W1, b1, W2, b2, b_g, n_shared, activation)
    T, d = x.shape
    E = W_g.shape[0]
    h = W1.shape[1]
    S = n_shared
    dev = x.device
    _check_b_sel(b_sel, E, dev)
    dt = _dtype_code(x)
    nbytes = moe_workspace_bytes(T, d, h, E, k, S, dt)
    if nbytes == 0:
        raise RuntimeError("invalid problem shape for moe_workspace_bytes")
    if noalloc:
        workspace = None
    elif workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=x.dtype, device=dev)
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    zl = torch.empty((1,), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    kept = torch.empty((E,), dtype=torch.int32, device=dev)
    slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)

    launch, keep = _launch(x, T, d, h, dt, b_g, workspace, zl, activation, min_capacity, stage_events, b_sel)
    launch.expert_counts = counts.data_ptr()
    launch.expert_kept = kept.data_ptr()
    launch.slot_pos = slot_pos.data_ptr()
    launch.weights_packed = 1 if weights_packed else 0
    ptr = lambda t: t.data_ptr() if t is not None else None
    call = moe_forward_noalloc if noalloc else moe_forward
    status = call(x.data_ptr(), W_g.data_ptr(), W1.data_ptr(), ptr(b1), W2.data_ptr(), ptr(b2), E, k,
                  float(capacity_factor), S, out.data_ptr(), topk_idx.data_ptr(), topk_w.data_ptr(),
                  aux.data_ptr(), launch)
    del keep
    if status != MOE_OK:
        raise RuntimeError(moe_status_string(status))
    return MoEOutput(out, topk_idx, topk_w, aux, zl, counts, kept, slot_pos)


@dataclass
class ExpertChoiceOutput:
    out: "object"            # [T, d], dtype of x
    ec_token: "object"       # [E, C] int32, ascending token order per expert
    ec_w: "object"           # [E, C] float32
    aux_loss: "object"       # [1] float32
    z_loss: "object"         # [1] float32


def expert_choice_capacity(capacity_factor: float, T: int, E: int, min_capacity: int = 0) -> int:
    """Tokens per expert from a capacity factor, as the library computes it
    (``moe_expert_choice_capacity``); raises ValueError for invalid arguments."""
    C = moe_expert_choice_capacity(float(capacity_factor), int(T), int(E), int(min_capacity))
    if C < 1:
        raise ValueError("expert choice needs a capacity factor > 0, T >= 1, E >= 1 and min_capacity >= 0")
    return C


def forward_expert_choice(x, W_g, W1, b1, W2, b2, C: int, n_shared: int = 0, b_g=None, *,
                          activation: str = "gelu", stage_events: Optional[Sequence] = None,
                          workspace=None, weights_packed: bool = False) -> ExpertChoiceOutput:
    """Run the layer with expert-choice routing (each expert takes its C
    best-scoring tokens) on torch tensors that live on one GPU.  Arguments as
    for ``forward``; C in 1..T."""
    import torch
    _check_tensors(x, W_g, W1, b1, W2, b2, b_g, n_shared, activation)
    T, d = x.shape
    E = W_g.shape[0]
    h = W1.shape[1]
    dt = _dtype_code(x)
    nbytes = moe_workspace_bytes_expert_choice(T, d, h, E, C, n_shared, dt)
    if nbytes == 0:
        raise RuntimeError("invalid problem shape for moe_workspace_bytes_expert_choice")
    dev = x.device
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=x.dtype, device=dev)
    ec_token = torch.empty((E, C), dtype=torch.int32, device=dev)
    ec_w = torch.empty((E, C), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    zl = torch.empty((1,), dtype=torch.float32, device=dev)
    launch, keep = _launch(x, T, d, h, dt, b_g, workspace, zl, activation, 0, stage_events)
    launch.weights_packed = 1 if weights_packed else 0
    ptr = lambda t: t.data_ptr() if t is not None else None
    status = moe_forward_expert_choice(x.data_ptr(), W_g.data_ptr(), W1.data_ptr(), ptr(b1), W2.data_ptr(),
                                       ptr(b2), E, C, n_shared, out.data_ptr(), ec_token.data_ptr(),
                                       ec_w.data_ptr(), aux.data_ptr(), launch)
    del keep
    if status != MOE_OK:
        raise RuntimeError(moe_status_string(status))
    return ExpertChoiceOutput(out, ec_token, ec_w, aux, zl)


def pack_weights(w):
    """The tile-packed layout (moe_pack_weights) of a contiguous bf16 expert
    weight [E+S, N, K] on a GPU, N and K multiples of 256: a new tensor of the
    same shape whose memory holds the packed blocks (for ``weights_packed``)."""
    import torch
    if w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous() or w.dim() != 3:
        raise ValueError("pack_weights takes a contiguous bf16 [E+S, N, K] tensor on a GPU")
    m, N, K = w.shape
    wp = torch.empty_like(w)
    st = moe_pack_weights(w.data_ptr(), m, N, K, MOE_BF16, wp.data_ptr(), torch.cuda.current_stream(w.device).cuda_stream)
    if st != MOE_OK:
        raise RuntimeError(moe_status_string(st))
    return wp


def quantize_mxfp8(w):
    """MXFP8 of a bf16 tensor on the GPU along its last dimension (a multiple of
    32): returns (codes uint8, same shape; scales uint8, last dimension / 32)."""
    import torch
    if w.dtype != torch.bfloat16 or not w.is_cuda or not w.is_contiguous():
        raise ValueError("quantize_mxfp8 takes a contiguous bf16 tensor on a GPU")
    cols = w.shape[-1]
    rows = w.numel() // cols
    codes = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    scales = torch.empty((*w.shape[:-1], cols // 32), dtype=torch.uint8, device=w.device)
    st = moe_quantize_mxfp8(w.data_ptr(), rows, cols, codes.data_ptr(), scales.data_ptr(),
                            torch.cuda.current_stream(w.device).cuda_stream)
    if st != MOE_OK:
        raise RuntimeError(moe_status_string(st))
    return codes, scales


def forward_mxfp8(x, W_g, W1, W1s, b1, W2, W2s, b2, k: int, capacity_factor: float = 0.0, n_shared: int = 0,
                  b_g=None, *, activation: str = "gelu", min_capacity: int = 0,
                  stage_events: Optional[Sequence] = None, workspace=None, b_sel=None) -> MoEOutput:
    """The layer with MXFP8 expert Linears: x, W_g, biases bf16; W1 / W2 as
    (codes, scales) from ``quantize_mxfp8`` of [E+S, h, d] / [E+S, d, h];
    b_g and b_sel as in ``forward``."""
    import torch
    for t in (x, W_g, b1, b2):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError("x, W_g, b1 and b2 of the MXFP8 layer must be bf16")
    for t in (W1, W1s, W2, W2s):
        if t.dtype != torch.uint8:
            raise ValueError("MXFP8 weight codes and scales must be uint8 (from quantize_mxfp8)")
    if activation not in ACTIVATIONS:
        raise ValueError(f"activation must be one of {sorted(ACTIVATIONS)}")
    T, d = x.shape
    E = W_g.shape[0]
    h = W1.shape[1]
    S = n_shared
    if W_g.shape != (E, d) or W1.shape != (E + S, h, d) or W1s.shape != (E + S, h, d // 32) or \
            W2.shape != (E + S, d, h) or W2s.shape != (E + S, d, h // 32) or \
            (b1 is not None and b1.shape != (E + S, h)) or (b2 is not None and b2.shape != (E + S, d)):
        raise ValueError("inconsistent MXFP8 layer shapes")
    for t in (x, W_g, W1, W1s, W2, W2s, b1, b2):
        if t is not None and (not t.is_cuda or t.device != x.device or not t.is_contiguous()):
            raise ValueError("all tensors must be contiguous on one GPU")
    dev = x.device
    if b_g is not None and (b_g.dtype != torch.float32 or b_g.shape != (E,) or b_g.device != dev
                            or not b_g.is_contiguous()):
        raise ValueError("b_g must be a contiguous float32 [E] on the same GPU")
    _check_b_sel(b_sel, E, dev)
    nbytes = moe_workspace_bytes_mxfp8(T, d, h, E, k, S)
    if nbytes == 0:
        raise RuntimeError("invalid problem shape for moe_workspace_bytes_mxfp8")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = torch.empty((T, d), dtype=x.dtype, device=dev)
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    aux = torch.empty((1,), dtype=torch.float32, device=dev)
    zl = torch.empty((1,), dtype=torch.float32, device=dev)
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    kept = torch.empty((E,), dtype=torch.int32, device=dev)
    slot_pos = torch.empty((T, k), dtype=torch.int32, device=dev)
    launch, keep = _launch(x, T, d, h, MOE_BF16, b_g, workspace, zl, activation, min_capacity, stage_events, b_sel)
    launch.expert_counts, launch.expert_kept, launch.slot_pos = counts.data_ptr(), kept.data_ptr(), slot_pos.data_ptr()
    ptr = lambda t: t.data_ptr() if t is not None else None
    status = moe_forward_mxfp8(x.data_ptr(), W_g.data_ptr(), W1.data_ptr(), W1s.data_ptr(), ptr(b1), W2.data_ptr(),
                               W2s.data_ptr(), ptr(b2), E, k, float(capacity_factor), S, out.data_ptr(),
                               topk_idx.data_ptr(), topk_w.data_ptr(), aux.data_ptr(), launch)
    del keep
    if status != MOE_OK:
        raise RuntimeError(moe_status_string(status))
    return MoEOutput(out, topk_idx, topk_w, aux, zl, counts, kept, slot_pos)


__all__ = ["forward", "MoEOutput", "moe_forward", "moe_workspace_bytes", "moe_status_string", "MoeLaunch",
           "forward_expert_choice", "ExpertChoiceOutput", "moe_forward_expert_choice",
           "moe_workspace_bytes_expert_choice", "expert_choice_capacity", "moe_expert_choice_capacity", "STAGES_EXPERT_CHOICE",
           "pack_weights", "moe_pack_weights", "quantize_mxfp8", "forward_mxfp8", "moe_quantize_mxfp8", "moe_workspace_bytes_mxfp8", "moe_forward_mxfp8",
           "moe_forward_noalloc", "MOE_ERR_SCRATCH", "MOE_NOALLOC_SCRATCH_BYTES", "ACTIVATIONS", "MOE_ACT_GELU", "MOE_ACT_SILU", "MOE_F32", "MOE_BF16", "MOE_OK", "MOE_ERR_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
           "MOE_ERR_HIP", "MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_MAX_SHARED", "MOE_NUM_STAGE_EVENTS",
           "STAGES", "EXPORTS", "LIB_PATH"]
