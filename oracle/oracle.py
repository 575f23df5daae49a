"""Python face of the fp64 CPU oracle (``attn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product package.  It shares no code
with the HIP path; both sides only share the seeded input generator.

Functions follow the X-Stage paper (arXiv 2607.23264): the attention is the
plain softmax-attention definition that FlashAttention computes exactly (up to
rounding), and the placement is the post-attention All-to-All of Fig. 5 on the
pith.science review page (steps d-e), read as: rank r owns heads
[r*H/P, (r+1)*H/P), destination rank p owns rows [p*S/P, (p+1)*S/P), and the
destination buffer is laid out [B][P][S/P][H][d].  The pre-attention exchange
(steps a-c) is read the same way in reverse: source rank p holds rows
[p*S/P, (p+1)*S/P) of all heads, the P chunks laid out [B][P][S/P][H][d].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
# UA_ORACLE_LIB points the loader at another build of attn_oracle.c (the
# mutation test compiles deliberately broken copies and runs the pins on them).
LIB_PATH = os.environ.get("UA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``attn_oracle.c`` into ``liboracle.so`` with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
               _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(LIB_PATH)
    i64, u16p, f64p, i64p = (ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
                             ctypes.POINTER(ctypes.c_double),
                             ctypes.POINTER(ctypes.c_int64))
    lib.oracle_widen.argtypes = [u16p, f64p, i64]
    lib.oracle_widen.restype = None
    lib.oracle_softmax_row.argtypes = [u16p, u16p, i64, i64, i64, ctypes.c_double,
                                       i64, i64, i64, f64p]
    lib.oracle_softmax_row.restype = ctypes.c_double
    lib.oracle_attn_rows.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64,
                                     ctypes.c_double, i64p, i64, f64p, ctypes.c_int]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = [ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_dest_offset.argtypes = [i64] * 9
    lib.oracle_dest_offset.restype = i64
    lib.oracle_dest_offsets.argtypes = [i64p, i64, i64, i64, i64, i64, i64, i64, i64p]
    lib.oracle_dest_offsets.restype = None
    lib.oracle_permute.argtypes = [u16p, i64, i64, i64, i64, i64, i64, u16p]
    lib.oracle_permute.restype = ctypes.c_int
    lib.oracle_gather.argtypes = [u16p, i64, i64, i64, i64, i64, i64, u16p]
    lib.oracle_gather.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle expects bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def _ptr(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values, same shape."""
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_widen(_ptr(bits, ctypes.c_uint16), _ptr(out, ctypes.c_double),
                         bits.size)
    return out


def softmax_row(Q, K, scale, b, h, s) -> np.ndarray:
    """Softmax weights over all keys j for query row (b, h, s); Q, K [B][S][Hl][d]."""
    Q, K = _u16(Q), _u16(K)
    B, S, Hl, d = Q.shape
    w = np.empty(S, dtype=np.float64)
    _load().oracle_softmax_row(_ptr(Q, ctypes.c_uint16), _ptr(K, ctypes.c_uint16),
                               S, Hl, d, float(scale), b, h, s,
                               _ptr(w, ctypes.c_double))
    return w


def attn_rows(Q, K, V, scale, rows, nthreads: int = 0) -> np.ndarray:
    """Attention output rows in fp64.

    Q, K, V: uint16 [B][S][Hl][d] (bf16 bits); rows: int64 [n][3] of (b, h_l, s).
    Returns float64 [n][d].
    """
    Q, K, V = _u16(Q), _u16(K), _u16(V)
    if not (Q.shape == K.shape == V.shape) or Q.ndim != 4:
        raise ValueError("Q, K, V must share one [B][S][Hl][d] shape")
    B, S, Hl, d = Q.shape
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    rc = _load().oracle_attn_rows(_ptr(Q, ctypes.c_uint16), _ptr(K, ctypes.c_uint16),
                                  _ptr(V, ctypes.c_uint16), B, S, Hl, d, float(scale),
                                  _ptr(rows, ctypes.c_int64), rows.shape[0],
                                  _ptr(out, ctypes.c_double), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows failed (row out of range or no memory)")
    return out


def attn_all(Q, K, V, scale, nthreads: int = 0) -> np.ndarray:
    """All rows; returns float64 [B][S][Hl][d] (the local, head-partitioned output)."""
    B, S, Hl, d = Q.shape
    bb, ss, hh = np.meshgrid(np.arange(B), np.arange(S), np.arange(Hl), indexing="ij")
    rows = np.stack([bb.ravel(), hh.ravel(), ss.ravel()], axis=1)
    return attn_rows(Q, K, V, scale, rows, nthreads).reshape(B, S, Hl, d)


def max_threads(nthreads: int = 0) -> int:
    return int(_load().oracle_max_threads(int(nthreads)))


def dest_offset(b, s, h_l, B, S, H, d, P, rank) -> int:
    """Element offset of row (b, s, h_l) in the [B][P][S/P][H][d] buffer, or -1."""
    return int(_load().oracle_dest_offset(b, s, h_l, B, S, H, d, P, rank))


def dest_offsets(rows, B, S, H, d, P, rank) -> np.ndarray:
    """Vector form of dest_offset; rows are (b, h_l, s) triples."""
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty(rows.shape[0], dtype=np.int64)
    _load().oracle_dest_offsets(_ptr(rows, ctypes.c_int64), rows.shape[0],
                                B, S, H, d, P, rank, _ptr(out, ctypes.c_int64))
    return out


def gather(X, H, P, rank) -> np.ndarray:
    """This rank's heads of the sequence-partitioned X [B][P][S/P][H][d] (or the
    same bytes as [B][S][H][d]) as X_local [B][S][Hl][d] (bit copy)."""
    X = _u16(X)
    if X.ndim == 5:
        B, P_, Sp, H_, d = X.shape
        S = P_ * Sp
    else:
        B, S, H_, d = X.shape
        P_ = P
    if H_ != H or P_ != P or H % P != 0:
        raise ValueError("shape mismatch between X, H and P")
    out = np.empty((B, S, H // P, d), dtype=np.uint16)
    rc = _load().oracle_gather(_ptr(X, ctypes.c_uint16), B, S, H, d, P, rank,
                               _ptr(out, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle_gather rejected its arguments")
    return out


def permute(O_local, H, P, rank, dest) -> None:
    """Bit copy of O_local [B][S][Hl][d] into dest [B][P][S/P][H][d] (in place)."""
    O_local = _u16(O_local)
    if not (isinstance(dest, np.ndarray) and dest.dtype == np.uint16
            and dest.flags["C_CONTIGUOUS"]):
        raise TypeError("dest must be a C-contiguous uint16 array")
    B, S, Hl, d = O_local.shape
    if Hl * P != H or dest.size != B * S * H * d:
        raise ValueError("shape mismatch between O_local, H, P and dest")
    rc = _load().oracle_permute(_ptr(O_local, ctypes.c_uint16), B, S, H, d, P, rank,
                                _ptr(dest, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle_permute rejected its arguments")
