"""GPU tests of the measurement entry points: the traced fused call (also in
its workspace form, on the key-split and stream-K launches) writes
bit-identical output plus sane timestamps, and the store-only epilogue kernel
writes exactly this rank's slots with its closed-form values."""
import numpy as np
import pytest

import comm_fusion_amd as ua
from gpu_helpers import sentinel_buffer, to_dev, to_host_bits
from ua_inputs import SENTINEL_BITS, make_qkv

pytestmark = pytest.mark.gpu

SHAPES = [
    # B, S, H, P, rank, d
    (1, 512, 4, 2, 0, 64),
    (2, 200, 8, 8, 3, 128),
    (1, 520, 64, 1, 0, 128),   # 8-wave workgroups
    (3, 129, 9, 3, 2, 64),
    (2, 1100, 64, 2, 1, 64),   # d = 64, two row blocks per wave on 32-key tiles
]


def _dev4(bits):
    return to_dev(bits).view(*bits.shape)


@pytest.mark.parametrize("B,S,H,P,rank,d", SHAPES)
def test_trace_build_output_is_bit_identical_and_timestamps_are_ordered(B, S, H, P, rank, d):
    import torch
    Q, K, V = make_qkv(B, S, H // P, d, 100 + S)
    q, k, v = _dev4(Q), _dev4(K), _dev4(V)
    ref = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused(q, k, v, rank, P, ref)
    n = ua.work_units(B, S, H, d, P)
    assert n > 0
    trace = torch.zeros(4 * n, dtype=torch.int64, device="cuda")
    got = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_trace(q, k, v, rank, P, got, trace)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host_bits(got), to_host_bits(ref))
    t = trace.cpu().numpy().reshape(n, 4)
    assert np.all(t[:, 0] > 0)
    assert np.all(t[:, 0] <= t[:, 1]) and np.all(t[:, 1] <= t[:, 2])
    assert np.all(t[:, 3] > 0)
    # shader clock implied by cycles over elapsed 100 MHz ticks (> 1 tick)
    span = t[:, 2] - t[:, 0]
    ok = span > 10
    mhz = t[ok, 3] / span[ok] * 100.0
    assert np.all((mhz > 200) & (mhz < 4000)), mhz


@pytest.mark.parametrize("B,S,H,P,rank,d", SHAPES)
def test_store_only_epilogue_writes_the_closed_form_into_owned_slots(B, S, H, P, rank, d):
    import torch
    dest = sentinel_buffer(B * S * H * d)
    ua.epilogue_store_only(B, S, H, d, rank, P, dest)
    torch.cuda.synchronize()
    got = to_host_bits(dest).reshape(B, S, H, d)   # [B][P][S/P][H][d] == [B][S][H][d]
    Hl = H // P
    s = np.arange(S, dtype=np.int64)[:, None, None]
    g = (rank * Hl + np.arange(Hl, dtype=np.int64))[None, :, None]
    c = np.arange(d, dtype=np.int64)[None, None, :]
    want = ((7 * s + 13 * g + 3 * c) & 0x3FFF).astype(np.uint16)
    for b in range(B):
        np.testing.assert_array_equal(got[b, :, rank * Hl:(rank + 1) * Hl], want)
    others = np.delete(got, np.s_[rank * Hl:(rank + 1) * Hl], axis=2)
    assert np.all(others == SENTINEL_BITS)


# B, S, H, P, rank, d: stream-K (the DiT-long shape), an equal split with key
# groups, a plain launch through the workspace form
SPLIT_TRACE_SHAPES = [(1, 16384, 24, 8, 5, 128), (1, 4096, 24, 8, 3, 128), (1, 512, 4, 2, 0, 64)]


@pytest.mark.parametrize("B,S,H,P,rank,d", SPLIT_TRACE_SHAPES)
def test_traced_workspace_call_is_bit_identical_with_one_record_per_workgroup(B, S, H, P, rank, d):
    import torch
    Q, K, V = make_qkv(B, S, H // P, d, 200 + S)
    q, k, v = _dev4(Q), _dev4(K), _dev4(V)
    ws = ua.new_workspace(B, S, H, d, P, q.device)
    ref = sentinel_buffer(B * S * H * d)
    if ws is None:
        ua.attn_ulysses_fused(q, k, v, rank, P, ref)
    else:
        ua.attn_ulysses_fused_ws(q, k, v, rank, P, ref, ws)
    n = ua.work_units(B, S, H, d, P, workspace=ws is not None)
    trace = torch.zeros(4 * n, dtype=torch.int64, device="cuda")
    got = sentinel_buffer(B * S * H * d)
    ua.attn_ulysses_fused_trace(q, k, v, rank, P, got, trace, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host_bits(got), to_host_bits(ref))
    t = trace.cpu().numpy().reshape(n, 4)
    assert np.all(t[:, 0] > 0) and np.all(t[:, 3] > 0)          # every workgroup recorded itself
    assert np.all(t[:, 0] <= t[:, 1]) and np.all(t[:, 1] <= t[:, 2])
    stored = int((t[:, 1] < t[:, 2]).sum())
    # every query tile is stored by exactly one workgroup: all of them in a
    # plain launch, one of the n_split of an equal split, and in stream-K the
    # one that merges (its query tiles are the plain launch's)
    n_split = ua.key_split(B, S, H, d, P) if ws is not None else 1
    if n_split == 1:
        assert stored == n
    elif ua.stream_k_iters(B, S, H, d, P):
        assert stored == ua.work_units(B, S, H, d, P)
    else:
        assert stored == n // n_split
    span = t[:, 2] - t[:, 0]
    ok = span > 10
    mhz = t[ok, 3] / span[ok] * 100.0
    assert np.all((mhz > 200) & (mhz < 4000)), mhz
