"""ctypes marshalling for the MoE expert path (see include/moe_combine.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels (moe_recv_layout is the library's host routine)."""
from __future__ import annotations

import ctypes

import numpy as np

from ._binding import UA_OK, UAError, _ptr, _stream, lib

MOE_EXPERT_WAVE = 0
MOE_INTERLEAVED = 1
MOE_MAX_WAVE = 32


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
                ("E", ctypes.c_int64), ("k", ctypes.c_int64)]


_set = False


def _lib():
    global _set
    L = lib()
    if not _set:
        vp, i, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        sp = ctypes.POINTER(MoeShape)
        L.moe_recv_layout.argtypes = [vp, i, i, sp, vp, vp, i64]
        L.moe_recv_layout.restype = i
        L.moe_experts_combine.argtypes = [vp, vp, vp, vp, vp, vp, i, sp, vp, vp, i, i, vp]
        L.moe_experts_combine.restype = i
        L.moe_experts_local.argtypes = [vp, vp, vp, vp, vp, vp, i, sp, vp, vp, i, vp]
        L.moe_experts_local.restype = i
        L.moe_combine_scatter.argtypes = [vp, vp, i64, i, sp, vp, vp]
        L.moe_combine_scatter.restype = i
        L.moe_workspace_bytes.argtypes = [i, sp]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_experts_combine_ws.argtypes = [vp, vp, vp, vp, vp, vp, i, sp, vp, vp, i, i, vp, ctypes.c_size_t, vp]
        L.moe_experts_combine_ws.restype = i
        L.moe_experts_local_ws.argtypes = [vp, vp, vp, vp, vp, vp, i, sp, vp, vp, i, vp, ctypes.c_size_t, vp]
        L.moe_experts_local_ws.restype = i
        _set = True
    return L


def moe_recv_layout(topk_idx: np.ndarray, rank: int, P: int, hidden: int, inter: int, E: int):
    """This rank's receive layout from host routing topk_idx [P][T][k] (int32):
    (expert_offsets int64 [E/P + 1], row_slot int32 [N])."""
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    Pp, T, k = idx.shape
    shp = MoeShape(T, hidden, inter, E, k)
    off = np.zeros(E // P + 1, np.int64)
    cap = max(idx.size, 1)
    slots = np.zeros(cap, np.int32)
    st = _lib().moe_recv_layout(idx.ctypes.data, int(rank), int(P), ctypes.byref(shp), off.ctypes.data,
                                slots.ctypes.data, cap)
    if st != UA_OK:
        raise UAError("moe_recv_layout", st)
    return off, slots[: off[-1]].copy()


def _check(name, t, dtype, numel=None):
    import torch
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous %s GPU tensor" % (name, dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))


def _shape(x, W1, W2, row_slot, topk_w, P, E, out, out_rows, act):
    """Checks dtypes and sizes of a call's tensors; returns its MoeShape."""
    import torch
    if x.dim() != 3 or W1.dim() != 3 or topk_w.dim() != 3:
        raise ValueError("x [P][T][hidden], W1 [E/P][2*inter][hidden] and topk_w [P][T][k] expected")
    Pp, T, hidden = (int(v) for v in x.shape)
    inter = int(W1.shape[1]) // 2
    k = int(topk_w.shape[-1])
    if Pp != P or tuple(topk_w.shape[:2]) != (P, T) or tuple(W1.shape) != (E // P, 2 * inter, hidden):
        raise ValueError("inconsistent x / topk_w / W1 shapes")
    N = int(row_slot.numel())
    _check("x", x, torch.bfloat16)
    _check("W1", W1, torch.bfloat16)
    _check("W2", W2, torch.bfloat16, (E // P) * hidden * inter)
    _check("row_slot", row_slot, torch.int32)
    _check("topk_w", topk_w, torch.float32)
    _check("out", out, torch.bfloat16, out_rows * hidden)
    _check("act", act, torch.bfloat16, N * inter)
    return MoeShape(T, hidden, inter, E, k)


def moe_experts_combine(x, row_slot, topk_w, expert_offsets, W1, W2, P, E, combine, act,
                        schedule=MOE_INTERLEAVED, experts_per_wave=4, stream=None):
    """x [P][T][hidden] bf16, row_slot int32 [N], topk_w float32 [P][T][k],
    expert_offsets host int64 [E/P + 1], W1 [E/P][2*inter][hidden], W2
    [E/P][hidden][inter] bf16, combine bf16 [P][T][k][hidden] (or flat), act
    bf16 workspace of N*inter elements (all torch tensors on one GPU)."""
    shp = _shape(x, W1, W2, row_slot, topk_w, P, E, combine,
                 P * int(x.shape[1]) * int(topk_w.shape[-1]), act)
    off = np.ascontiguousarray(expert_offsets, dtype=np.int64)
    if off.shape != (E // P + 1,) or int(off[-1]) != row_slot.numel():
        raise ValueError("expert_offsets must hold E/P + 1 offsets ending at len(row_slot)")
    st = _lib().moe_experts_combine(_ptr(x), _ptr(row_slot), _ptr(topk_w), off.ctypes.data, _ptr(W1), _ptr(W2),
                                    int(P), ctypes.byref(shp), _ptr(combine), _ptr(act), int(schedule),
                                    int(experts_per_wave), _stream(stream, x, W1, W2, combine, act))
    if st != UA_OK:
        raise UAError("moe_experts_combine", st)


def moe_workspace_bytes(P, T, hidden, inter, E, k) -> int:
    """Bytes of the persistent form's workspace for this shape (0 if invalid)."""
    return int(_lib().moe_workspace_bytes(int(P), ctypes.byref(MoeShape(T, hidden, inter, E, k))))


def new_moe_workspace(x, W1, topk_w, P, E):
    """A uint8 device tensor of moe_workspace_bytes for the call's shape."""
    import torch
    T, hidden = int(x.shape[1]), int(x.shape[2])
    n = moe_workspace_bytes(P, T, hidden, int(W1.shape[1]) // 2, E, int(topk_w.shape[-1]))
    return torch.empty(n, dtype=torch.uint8, device=x.device)


def _ws(workspace):
    import torch
    if workspace is None or not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous GPU tensor")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def moe_experts_combine_ws(x, row_slot, topk_w, expert_offsets, W1, W2, P, E, combine, act, workspace,
                           schedule=MOE_INTERLEAVED, experts_per_wave=4, stream=None):
    """moe_experts_combine in the persistent form; workspace from new_moe_workspace."""
    shp = _shape(x, W1, W2, row_slot, topk_w, P, E, combine,
                 P * int(x.shape[1]) * int(topk_w.shape[-1]), act)
    off = np.ascontiguousarray(expert_offsets, dtype=np.int64)
    if off.shape != (E // P + 1,) or int(off[-1]) != row_slot.numel():
        raise ValueError("expert_offsets must hold E/P + 1 offsets ending at len(row_slot)")
    wp, wb = _ws(workspace)
    st = _lib().moe_experts_combine_ws(_ptr(x), _ptr(row_slot), _ptr(topk_w), off.ctypes.data, _ptr(W1), _ptr(W2),
                                       int(P), ctypes.byref(shp), _ptr(combine), _ptr(act), int(schedule),
                                       int(experts_per_wave), wp, wb, _stream(stream, x, W1, W2, combine, act))
    if st != UA_OK:
        raise UAError("moe_experts_combine_ws", st)


def moe_experts_local_ws(x, row_slot, topk_w, expert_offsets, W1, W2, P, E, y_local, act, workspace,
                         experts_per_wave=4, stream=None):
    """moe_experts_local in the persistent form."""
    shp = _shape(x, W1, W2, row_slot, topk_w, P, E, y_local, row_slot.numel(), act)
    off = np.ascontiguousarray(expert_offsets, dtype=np.int64)
    if off.shape != (E // P + 1,) or int(off[-1]) != row_slot.numel():
        raise ValueError("expert_offsets must hold E/P + 1 offsets ending at len(row_slot)")
    wp, wb = _ws(workspace)
    st = _lib().moe_experts_local_ws(_ptr(x), _ptr(row_slot), _ptr(topk_w), off.ctypes.data, _ptr(W1), _ptr(W2),
                                     int(P), ctypes.byref(shp), _ptr(y_local), _ptr(act), int(experts_per_wave),
                                     wp, wb, _stream(stream, x, W1, W2, y_local, act))
    if st != UA_OK:
        raise UAError("moe_experts_local_ws", st)


def moe_experts_local(x, row_slot, topk_w, expert_offsets, W1, W2, P, E, y_local, act,
                      experts_per_wave=4, stream=None):
    """The serial form's expert half: row i's weighted output into y_local [N][hidden]."""
    shp = _shape(x, W1, W2, row_slot, topk_w, P, E, y_local, row_slot.numel(), act)
    off = np.ascontiguousarray(expert_offsets, dtype=np.int64)
    if off.shape != (E // P + 1,) or int(off[-1]) != row_slot.numel():
        raise ValueError("expert_offsets must hold E/P + 1 offsets ending at len(row_slot)")
    st = _lib().moe_experts_local(_ptr(x), _ptr(row_slot), _ptr(topk_w), off.ctypes.data, _ptr(W1), _ptr(W2),
                                  int(P), ctypes.byref(shp), _ptr(y_local), _ptr(act), int(experts_per_wave),
                                  _stream(stream, x, W1, W2, y_local, act))
    if st != UA_OK:
        raise UAError("moe_experts_local", st)


def moe_combine_scatter(y_local, row_slot, N, P, T, hidden, inter, E, k, combine, stream=None):
    """The serial form's exchange half: row i of y_local into slot row_slot[i]."""
    shp = MoeShape(T, hidden, inter, E, k)
    st = _lib().moe_combine_scatter(_ptr(y_local), _ptr(row_slot), int(N), int(P), ctypes.byref(shp),
                                    _ptr(combine), _stream(stream, y_local, combine))
    if st != UA_OK:
        raise UAError("moe_combine_scatter", st)
