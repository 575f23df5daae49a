"""ctypes marshalling for libulysses_attn.so (see include/ulysses_attn.h)."""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libulysses_attn.so")

UA_OK = 0
UA_ERR_NULL = -1
UA_ERR_SHAPE = -2
UA_ERR_RANK = -3
UA_ERR_ALIGN = -4
UA_ERR_UNSUPPORTED = -5
UA_ERR_HIP = -6
UA_ERR_WORKSPACE = -7
UA_ERR_SCRATCH = -8
SCRATCH_BYTES = 128 << 20   # UA_SCRATCH_BYTES: fixed device scratch of attn_ulysses_fused_noalloc


class UAError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (call, status_string(status), status))


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S", ctypes.c_int64),
                ("H", ctypes.c_int64), ("d", ctypes.c_int64)]


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded C library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libulysses_attn.so is not built (%s); run "
                          "`python -m comm_fusion_amd.build` or __graft_entry__.build()" % _LIB_PATH)
    # torch carries its own copy of the HIP runtime, which its libraries load
    # under another file name than ours asks for (same SONAME).  Loaded first,
    # that copy also satisfies this library's dependency; loaded after it, a
    # second runtime would come in, and torch's device pointers and streams
    # would be foreign to the one the library launches on.
    import torch  # noqa: F401
    L = ctypes.CDLL(_LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sp = ctypes.POINTER(Shape)
    L.attn_ulysses_fused.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp]
    L.attn_ulysses_fused.restype = i
    L.attn_ulysses_fused_noalloc.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp]
    L.attn_ulysses_fused_noalloc.restype = i
    L.attn_serial.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp]
    L.attn_serial.restype = i
    L.a2a_permute.argtypes = [vp, i, i, vp, sp, vp]
    L.a2a_permute.restype = i
    L.ua_status_string.argtypes = [i]
    L.ua_status_string.restype = ctypes.c_char_p
    L.ua_dest_bytes.argtypes = [sp]
    L.ua_dest_bytes.restype = ctypes.c_size_t
    L.ua_local_bytes.argtypes = [sp, i]
    L.ua_local_bytes.restype = ctypes.c_size_t
    L.ua_version.argtypes = []
    L.ua_version.restype = i
    L.attn_ulysses_fused_trace.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp, vp]
    L.attn_ulysses_fused_trace.restype = i
    L.ua_epilogue_store_only.argtypes = [i, i, vp, sp, vp]
    L.ua_epilogue_store_only.restype = i
    L.ua_work_units.argtypes = [sp, i]
    L.ua_work_units.restype = ctypes.c_int64
    L.ua_work_units_ws.argtypes = [sp, i]
    L.ua_work_units_ws.restype = ctypes.c_int64
    L.attn_ulysses_fused_trace_ws.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp, ctypes.c_size_t, vp, vp]
    L.attn_ulysses_fused_trace_ws.restype = i
    L.attn_ulysses_fused_io.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp]
    L.attn_ulysses_fused_io.restype = i
    L.a2a_gather.argtypes = [vp, i, i, vp, sp, vp]
    L.a2a_gather.restype = i
    sz = ctypes.c_size_t
    L.attn_ulysses_fused_ws.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp, sz, vp]
    L.attn_ulysses_fused_ws.restype = i
    L.attn_serial_ws.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp, sz, vp]
    L.attn_serial_ws.restype = i
    L.attn_ulysses_fused_io_ws.argtypes = [vp, vp, vp, i, i, vp, sp, f, vp, sz, vp]
    L.attn_ulysses_fused_io_ws.restype = i
    L.ua_workspace_bytes.argtypes = [sp, i]
    L.ua_workspace_bytes.restype = sz
    L.ua_workspace_count_bytes.argtypes = [sp, i]
    L.ua_workspace_count_bytes.restype = sz
    L.ua_key_split.argtypes = [sp, i]
    L.ua_key_split.restype = i
    L.ua_stream_k_iters.argtypes = [sp, i]
    L.ua_stream_k_iters.restype = ctypes.c_int64
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().ua_status_string(int(status)).decode()


def version() -> int:
    return int(lib().ua_version())


def dest_bytes(B, S, H, d) -> int:
    return int(lib().ua_dest_bytes(ctypes.byref(Shape(B, S, H, d))))


def local_bytes(B, S, H, d, P) -> int:
    return int(lib().ua_local_bytes(ctypes.byref(Shape(B, S, H, d)), int(P)))


def _ptr(t) -> int:
    return int(t.data_ptr()) if t is not None else 0


def _check_bf16(name, t, numel=None):
    import torch
    if t is None:
        return
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise TypeError("%s must be a contiguous bfloat16 GPU tensor" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))


def _stream(stream, *tensors) -> int:
    """The stream handle for a call on ``tensors``: they must share one device,
    and a torch stream passed in must belong to it; None means that device's
    current stream.  A raw handle (int) is taken as given."""
    import torch
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError("all tensors of a call must be on one device, got %s" % sorted(map(str, devs)))
    dev = devs.pop() if devs else None
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif dev is not None and hasattr(stream, "device") and torch.device(stream.device) != dev:
        raise ValueError("stream is on %s but the tensors are on %s" % (stream.device, dev))
    return int(getattr(stream, "cuda_stream", stream))


def _qkv_shape(Q, K, V, P):
    if Q.dim() != 4 or tuple(K.shape) != tuple(Q.shape) or tuple(V.shape) != tuple(Q.shape):
        raise ValueError("Q, K, V must share one [B][S][Hl][d] shape")
    B, S, Hl, d = (int(x) for x in Q.shape)
    return Shape(B, S, Hl * int(P), d)


def attn_ulysses_fused(Q, K, V, rank, P, out, scale=None, stream=None):
    """Fused attention + post-attention All-to-All into ``out`` [B][P][S/P][H][d]."""
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_ulysses_fused(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out),
                                  ctypes.byref(shp), scale, _stream(stream, Q, K, V, out))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused", st)


def attn_serial(Q, K, V, rank, P, O_local, scale=None, stream=None):
    """Attention only, into the head-partitioned ``O_local`` [B][S][Hl][d]."""
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("O_local", O_local, Q.numel())
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_serial(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(O_local),
                           ctypes.byref(shp), scale, _stream(stream, Q, K, V, O_local))
    if st != UA_OK:
        raise UAError("attn_serial", st)


def a2a_permute(O_local, rank, P, out, stream=None):
    """Serial All-to-All: copy ``O_local`` rows into their slots of ``out``."""
    if O_local.dim() != 4:
        raise ValueError("O_local must be [B][S][Hl][d]")
    B, S, Hl, d = (int(x) for x in O_local.shape)
    shp = Shape(B, S, Hl * int(P), d)
    _check_bf16("O_local", O_local)
    _check_bf16("out", out, B * S * Hl * int(P) * d)
    st = lib().a2a_permute(_ptr(O_local), int(rank), int(P), _ptr(out), ctypes.byref(shp),
                           _stream(stream, O_local, out))
    if st != UA_OK:
        raise UAError("a2a_permute", st)


def _seq_shape(X, P):
    """Shape of a sequence-partitioned input, [B][P][S/P][H][d] or (the same
    bytes) [B][S][H][d]."""
    if X.dim() == 5:
        B, P_, Sp, H, d = (int(x) for x in X.shape)
        if P_ != int(P):
            raise ValueError("X has %d regions, expected P = %d" % (P_, int(P)))
        return Shape(B, P_ * Sp, H, d)
    if X.dim() == 4:
        B, S, H, d = (int(x) for x in X.shape)
        return Shape(B, S, H, d)
    raise ValueError("X must be [B][P][S/P][H][d] or [B][S][H][d]")


def attn_ulysses_fused_io(Xq, Xk, Xv, rank, P, out, scale=None, stream=None):
    """Both exchanges fused: this rank's heads read in place from the
    sequence-partitioned ``Xq, Xk, Xv``, output into ``out`` [B][P][S/P][H][d]."""
    shp = _seq_shape(Xq, P)
    n = shp.B * shp.S * shp.H * shp.d
    for nm, t in (("Xq", Xq), ("Xk", Xk), ("Xv", Xv)):
        _check_bf16(nm, t, n)
    _check_bf16("out", out, n)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_ulysses_fused_io(_ptr(Xq), _ptr(Xk), _ptr(Xv), int(rank), int(P), _ptr(out),
                                     ctypes.byref(shp), scale, _stream(stream, Xq, Xk, Xv, out))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused_io", st)


def a2a_gather(X, rank, P, X_local, stream=None):
    """Serial pre-attention All-to-All: this rank's heads of ``X`` into
    ``X_local`` [B][S][Hl][d]."""
    shp = _seq_shape(X, P)
    _check_bf16("X", X, shp.B * shp.S * shp.H * shp.d)
    _check_bf16("X_local", X_local, shp.B * shp.S * (shp.H // int(P)) * shp.d)
    st = lib().a2a_gather(_ptr(X), int(rank), int(P), _ptr(X_local), ctypes.byref(shp), _stream(stream, X, X_local))
    if st != UA_OK:
        raise UAError("a2a_gather", st)


def work_units(B, S, H, d, P, workspace=False) -> int:
    """Workgroups of the launch without (or, with workspace=True, with) a workspace."""
    fn = lib().ua_work_units_ws if workspace else lib().ua_work_units
    return int(fn(ctypes.byref(Shape(B, S, H, d)), int(P)))


def attn_ulysses_fused_trace(Q, K, V, rank, P, out, trace, scale=None, stream=None, workspace=None):
    """Measurement build of attn_ulysses_fused (or, given a workspace, of
    attn_ulysses_fused_ws); ``trace`` is an int64 GPU tensor of
    work_units(..., workspace=...) * 4 elements (see the C header)."""
    import torch
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    fn = lib().ua_work_units_ws if workspace is not None else lib().ua_work_units
    n_units = int(fn(ctypes.byref(shp), int(P)))
    if trace.dtype != torch.int64 or not trace.is_cuda or not trace.is_contiguous() \
            or trace.numel() != 4 * n_units:
        raise TypeError("trace must be a contiguous int64 GPU tensor of %d elements" % (4 * n_units))
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    if workspace is None:
        st = lib().attn_ulysses_fused_trace(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out),
                                            ctypes.byref(shp), scale, _stream(stream, Q, K, V, out, trace),
                                            _ptr(trace))
    else:
        wp, wb = _ws(workspace)
        st = lib().attn_ulysses_fused_trace_ws(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out),
                                               ctypes.byref(shp), scale, wp, wb,
                                               _stream(stream, Q, K, V, out, trace, workspace), _ptr(trace))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused_trace", st)


def epilogue_store_only(B, S, H, d, rank, P, out, stream=None):
    """The fused call's epilogue stores alone (closed-form values) into ``out``."""
    shp = Shape(int(B), int(S), int(H), int(d))
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    st = lib().ua_epilogue_store_only(int(rank), int(P), _ptr(out), ctypes.byref(shp), _stream(stream, out))
    if st != UA_OK:
        raise UAError("ua_epilogue_store_only", st)


def workspace_bytes(B, S, H, d, P) -> int:
    """Workspace bytes the *_ws calls need for this shape (0: no key split)."""
    return int(lib().ua_workspace_bytes(ctypes.byref(Shape(B, S, H, d)), int(P)))


def workspace_count_bytes(B, S, H, d, P) -> int:
    """Leading workspace bytes that hold the arrival counts (zero between calls)."""
    return int(lib().ua_workspace_count_bytes(ctypes.byref(Shape(B, S, H, d)), int(P)))


def stream_k_iters(B, S, H, d, P) -> int:
    """(query tile, key tile) iterations per workgroup of a stream-K split in
    the *_ws calls (0: the plain key split, or none)."""
    return int(lib().ua_stream_k_iters(ctypes.byref(Shape(B, S, H, d)), int(P)))


def key_split(B, S, H, d, P) -> int:
    """Workgroups that share each query tile's keys in a *_ws call (1: none)."""
    return int(lib().ua_key_split(ctypes.byref(Shape(B, S, H, d)), int(P)))


def new_workspace(B, S, H, d, P, device):
    """A zeroed workspace for the *_ws calls on ``device`` (a uint8 tensor), or
    None when the shape needs none."""
    import torch
    n = workspace_bytes(B, S, H, d, P)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def _ws(workspace):
    """(pointer, bytes) of a workspace tensor, or (0, 0) for None."""
    if workspace is None:
        return 0, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise TypeError("workspace must be a contiguous GPU tensor")
    return int(workspace.data_ptr()), int(workspace.numel() * workspace.element_size())


def attn_ulysses_fused_ws(Q, K, V, rank, P, out, workspace, scale=None, stream=None):
    """attn_ulysses_fused with a workspace (see new_workspace): shapes with fewer
    query tiles than CUs split each tile's keys over several workgroups."""
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    wp, wb = _ws(workspace)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_ulysses_fused_ws(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out),
                                     ctypes.byref(shp), scale, wp, wb, _stream(stream, Q, K, V, out, workspace))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused_ws", st)


def attn_serial_ws(Q, K, V, rank, P, O_local, workspace, scale=None, stream=None):
    """attn_serial with a workspace (see new_workspace)."""
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("O_local", O_local, Q.numel())
    wp, wb = _ws(workspace)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_serial_ws(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(O_local),
                              ctypes.byref(shp), scale, wp, wb, _stream(stream, Q, K, V, O_local, workspace))
    if st != UA_OK:
        raise UAError("attn_serial_ws", st)


def attn_ulysses_fused_io_ws(Xq, Xk, Xv, rank, P, out, workspace, scale=None, stream=None):
    """attn_ulysses_fused_io with a workspace (see new_workspace)."""
    shp = _seq_shape(Xq, P)
    n = shp.B * shp.S * shp.H * shp.d
    for nm, t in (("Xq", Xq), ("Xk", Xk), ("Xv", Xv)):
        _check_bf16(nm, t, n)
    _check_bf16("out", out, n)
    wp, wb = _ws(workspace)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_ulysses_fused_io_ws(_ptr(Xq), _ptr(Xk), _ptr(Xv), int(rank), int(P), _ptr(out),
                                        ctypes.byref(shp), scale, wp, wb,
                                        _stream(stream, Xq, Xk, Xv, out, workspace))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused_io_ws", st)


def attn_ulysses_fused_noalloc(Q, K, V, rank, P, out, scale=None, stream=None):
    """attn_ulysses_fused_ws with the workspace in the library's fixed device
    scratch (SCRATCH_BYTES per GPU): allocates nothing.  Calls that overlap on
    one GPU race on the scratch."""
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    st = lib().attn_ulysses_fused_noalloc(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out),
                                          ctypes.byref(shp), scale, _stream(stream, Q, K, V, out))
    if st != UA_OK:
        raise UAError("attn_ulysses_fused_noalloc", st)


def fused_write_counts(Q, K, V, rank, P, out, counts, workspace=None, scale=None, stream=None):
    """Write check: attn_ulysses_fused_ws (or the plain call) that also adds 1
    to counts[c] (int32 tensor of out.numel() // 8 entries, zeroed) for every
    16-byte chunk c of out it stores."""
    import torch
    shp = _qkv_shape(Q, K, V, P)
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _check_bf16(n, t)
    _check_bf16("out", out, shp.B * shp.S * shp.H * shp.d)
    if counts.dtype != torch.int32 or not counts.is_cuda or counts.numel() != out.numel() // 8:
        raise TypeError("counts must be an int32 GPU tensor of out.numel() // 8 elements")
    wp, wb = _ws(workspace)
    scale = 1.0 / math.sqrt(shp.d) if scale is None else float(scale)
    L = lib()
    L.ua_fused_write_counts.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                                  ctypes.POINTER(Shape), ctypes.c_float,
                                                                  ctypes.c_void_p, ctypes.c_size_t,
                                                                  ctypes.c_void_p, ctypes.c_void_p]
    L.ua_fused_write_counts.restype = ctypes.c_int
    st = L.ua_fused_write_counts(_ptr(Q), _ptr(K), _ptr(V), int(rank), int(P), _ptr(out), ctypes.byref(shp),
                                 scale, wp, wb, _stream(stream, Q, K, V, out, counts), _ptr(counts))
    if st != UA_OK:
        raise UAError("ua_fused_write_counts", st)
