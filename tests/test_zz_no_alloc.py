"""GPU check of attn_ulysses_fused_noalloc, the call that allocates nothing:
its key-split workspace lives in the library's fixed device scratch.

Through the C ABI, two calls in a row -- the DiT-long shape (4-way key split,
~99 MiB of scratch) and then the smaller DiT-image shape (2-way split) --
must each write exactly the bytes attn_ulysses_fused_ws writes with a fresh
workspace, and match the fp64 oracle on the sampled rows with the layout
exact.  A shape that needs no split must equal attn_ulysses_fused.
"""
import ctypes
import dataclasses
import math

import numpy as np
import pytest

import comm_fusion_amd as ua
import oracle
from comm_fusion_amd._binding import Shape
from gpu_helpers import assert_close, bits_to_f64, check_dest_layout, sentinel_buffer, to_dev, to_host_bits
from ua_inputs import WORKLOADS, sampled_rows, workload_qkv

pytestmark = pytest.mark.gpu


def _noalloc_c(q, k, v, w, dest):
    import torch
    shp = Shape(w.B, w.S, w.H, w.d)
    st = ua.lib().attn_ulysses_fused_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), w.rank, w.P,
                                             dest.data_ptr(), ctypes.byref(shp), 1.0 / math.sqrt(w.d),
                                             torch.cuda.current_stream().cuda_stream)
    assert st == ua.UA_OK, ua.status_string(st)


def _run(w):
    import torch
    Q, K, V = workload_qkv(w)
    q, k, v = (to_dev(x).view(*x.shape) for x in (Q, K, V))
    n = w.B * w.S * w.H * w.d
    got = sentinel_buffer(n)
    _noalloc_c(q, k, v, w, got)
    ref = sentinel_buffer(n)
    if ua.key_split(w.B, w.S, w.H, w.d, w.P) > 1:
        ws = ua.new_workspace(w.B, w.S, w.H, w.d, w.P, q.device)
        ua.attn_ulysses_fused_ws(q, k, v, w.rank, w.P, ref, ws)
    else:
        ua.attn_ulysses_fused(q, k, v, w.rank, w.P, ref)
    torch.cuda.synchronize()
    g, r = to_host_bits(got), to_host_bits(ref)
    np.testing.assert_array_equal(g, r)
    check_dest_layout(g, w.B, w.S, w.H, w.d, w.P, w.rank)
    rows = sampled_rows(dataclasses.replace(w, sampled=True))
    vals = oracle.attn_rows(Q, K, V, 1.0 / math.sqrt(w.d), rows)
    offs = oracle.dest_offsets(rows, w.B, w.S, w.H, w.d, w.P, w.rank)
    assert_close(bits_to_f64(g[offs[:, None] + np.arange(w.d)[None, :]]), vals, w.name)


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    big, small = WORKLOADS["dit_long"], WORKLOADS["dit_image"]
    for w in (big, small):
        assert ua.key_split(w.B, w.S, w.H, w.d, w.P) > 1
        assert 0 < ua.workspace_bytes(w.B, w.S, w.H, w.d, w.P) <= ua.SCRATCH_BYTES
    assert ua.workspace_bytes(small.B, small.S, small.H, small.d, small.P) < \
        ua.workspace_bytes(big.B, big.S, big.H, big.d, big.P)
    print("noalloc: dit_long then dit_image", flush=True)
    _run(big)
    _run(small)


def test_noalloc_without_a_split_equals_the_plain_call():
    w = WORKLOADS["tiny"]
    assert ua.key_split(w.B, w.S, w.H, w.d, w.P) == 1
    print("noalloc: tiny (no split)", flush=True)
    _run(w)
