"""The C-ABI library loads, exports every symbol its header declares, and
validates arguments on the host before any device access (CPU only: no call
here reaches a launch)."""
import ctypes
import os
import re

import pytest

import comm_fusion_amd as ua
from comm_fusion_amd._binding import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ulysses_attn.h")

A = 0x10000       # 16-byte aligned fake device addresses (never dereferenced:
B_ = 0x20000      # every call below fails validation first)
C = 0x30000
O = 0x40000


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert set(names) >= {"attn_ulysses_fused", "attn_serial", "a2a_permute", "ua_status_string",
                          "ua_dest_bytes", "ua_local_bytes", "ua_version"}
    L = ctypes.CDLL(ua.lib_path())
    for n in names:
        assert hasattr(L, n), "missing export %s" % n


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in [("UA_OK", 0), ("UA_ERR_NULL", -1), ("UA_ERR_SHAPE", -2), ("UA_ERR_RANK", -3),
                      ("UA_ERR_ALIGN", -4), ("UA_ERR_UNSUPPORTED", -5), ("UA_ERR_HIP", -6),
                      ("UA_ERR_WORKSPACE", -7), ("UA_ERR_SCRATCH", -8)]:
        assert re.search(r"\b%s\s*=\s*%d\b" % (name, val), text)
        assert getattr(ua, name) == val
        assert ua.status_string(val) and ua.status_string(val) != "unknown status"
    assert ua.status_string(12345) == "unknown status"
    assert ua.version() == 10200


def _fused(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125):
    L = ua.lib()
    return L.attn_ulysses_fused(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale, None)


def _serial(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125):
    L = ua.lib()
    return L.attn_serial(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale, None)


def _fused_io(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125):
    L = ua.lib()
    return L.attn_ulysses_fused_io(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale, None)


W = 0x1000000     # fake workspace address (16-byte aligned)


def _fused_ws(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125, ws=W, ws_bytes=1 << 40):
    return ua.lib().attn_ulysses_fused_ws(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale,
                                          ws, ws_bytes, None)


def _serial_ws(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125, ws=W, ws_bytes=1 << 40):
    return ua.lib().attn_serial_ws(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale,
                                   ws, ws_bytes, None)


def _fused_io_ws(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, scale=0.125, ws=W, ws_bytes=1 << 40):
    return ua.lib().attn_ulysses_fused_io_ws(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale,
                                             ws, ws_bytes, None)


def _permute(shape, rank=0, P=2, src=A, out=O):
    return ua.lib().a2a_permute(src, rank, P, out, ctypes.byref(Shape(*shape)), None)


def _gather(shape, rank=0, P=2, src=A, out=O):
    return ua.lib().a2a_gather(src, rank, P, out, ctypes.byref(Shape(*shape)), None)


@pytest.mark.parametrize("call", [_fused, _serial, _fused_io, _fused_ws, _serial_ws, _fused_io_ws])
def test_attention_argument_validation(call):
    good = (1, 64, 4, 64)
    assert ua.lib().attn_ulysses_fused(A, B_, C, 0, 2, O, None, 0.1, None) == ua.UA_ERR_NULL
    assert call(good, q=0) == ua.UA_ERR_NULL
    assert call(good, out=0) == ua.UA_ERR_NULL
    assert call((1, 63, 4, 64)) == ua.UA_ERR_SHAPE        # S % P
    assert call((1, 64, 5, 64)) == ua.UA_ERR_SHAPE        # H % P
    assert call((-1, 64, 4, 64)) == ua.UA_ERR_SHAPE
    assert call((1, 64, 0, 64)) == ua.UA_ERR_SHAPE
    assert call(good, P=0) == ua.UA_ERR_SHAPE
    assert call((1 << 40, 1 << 20, 4, 64)) == ua.UA_ERR_SHAPE  # byte size overflows
    assert call(good, rank=2) == ua.UA_ERR_RANK
    assert call(good, rank=-1) == ua.UA_ERR_RANK
    assert call(good, k=B_ + 8) == ua.UA_ERR_ALIGN
    assert call(good, out=O + 2) == ua.UA_ERR_ALIGN
    assert call((1, 64, 4, 96)) == ua.UA_ERR_UNSUPPORTED
    assert call(good, scale=0.0) == ua.UA_ERR_UNSUPPORTED
    assert call(good, scale=-1.0) == ua.UA_ERR_UNSUPPORTED
    assert call(good, scale=float("nan")) == ua.UA_ERR_UNSUPPORTED
    assert call(good, scale=float("inf")) == ua.UA_ERR_UNSUPPORTED
    assert call((1, 1 << 30, 8, 128), P=1) == ua.UA_ERR_UNSUPPORTED  # beyond grid limits
    assert call((1, 1, 1 << 18, 128), P=1) == ua.UA_ERR_UNSUPPORTED  # row stride Hl*d > 2^24
    assert call((0, 1, 1 << 18, 128), P=1) == ua.UA_ERR_UNSUPPORTED  # limits come before "empty"
    assert call((0, 1, 1 << 17, 128), P=1) == ua.UA_OK  # Hl*d = 2^24 is allowed


@pytest.mark.parametrize("call", [_fused, _serial, _fused_io, _fused_ws, _serial_ws, _fused_io_ws,
                                  _permute, _gather])
def test_empty_calls_succeed_without_touching_memory(call):
    copy = call in (_permute, _gather)
    assert call((0, 64, 4, 64), src=0, out=0) == ua.UA_OK if copy else \
        call((0, 64, 4, 64), q=0, k=0, v=0, out=0) == ua.UA_OK
    assert call((3, 0, 4, 128), src=0, out=0) == ua.UA_OK if copy else \
        call((3, 0, 4, 128), q=0, k=0, v=0, out=0) == ua.UA_OK


@pytest.mark.parametrize("call", [_permute, _gather])
def test_exchange_copy_argument_validation(call):
    good = (2, 64, 8, 128)
    assert call(good, src=0) == ua.UA_ERR_NULL
    assert call(good, out=0) == ua.UA_ERR_NULL
    assert call((2, 60, 8, 128), P=8) == ua.UA_ERR_SHAPE
    assert call(good, rank=5, P=4) == ua.UA_ERR_RANK
    assert call(good, src=A + 4) == ua.UA_ERR_ALIGN
    assert call(good, out=O + 8) == ua.UA_ERR_ALIGN
    assert call((2, 64, 8, 32)) == ua.UA_ERR_UNSUPPORTED


def test_fused_io_limits_the_full_row_stride():
    # Hl*d = 2^24 passes every call; H*d = 2^25 is beyond the in-place read of
    # the sequence-partitioned input, so only attn_ulysses_fused_io rejects it
    shape = (0, 2, 1 << 18, 128)
    assert _fused(shape, q=0, k=0, v=0, out=0) == ua.UA_OK
    assert _fused_io(shape, q=0, k=0, v=0, out=0) == ua.UA_ERR_UNSUPPORTED
    assert _fused_io((0, 2, 1 << 17, 128), q=0, k=0, v=0, out=0) == ua.UA_OK


def test_buffer_size_helpers():
    assert ua.dest_bytes(2, 32768, 24, 64) == 2 * 32768 * 24 * 64 * 2
    assert ua.local_bytes(2, 32768, 24, 64, 4) == 2 * 32768 * 6 * 64 * 2
    assert ua.local_bytes(1, 8, 5, 64, 2) == 0     # H % P != 0
    assert ua.dest_bytes(-1, 8, 4, 64) == 0
    assert ua.lib().ua_dest_bytes(None) == 0


def _trace(shape, rank=0, P=2, q=A, k=B_, v=C, out=O, trace=0x50000, scale=0.125):
    return ua.lib().attn_ulysses_fused_trace(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale,
                                             None, trace)


def _store_only(shape, rank=0, P=2, out=O):
    return ua.lib().ua_epilogue_store_only(rank, P, out, ctypes.byref(Shape(*shape)), None)


def test_measurement_entry_points_validate_like_the_fused_call():
    good = (1, 64, 4, 64)
    assert _trace(good, trace=0) == ua.UA_ERR_NULL
    assert _trace(good, trace=0x50008) == ua.UA_ERR_ALIGN
    assert _trace(good, q=0) == ua.UA_ERR_NULL
    assert _trace((1, 63, 4, 64)) == ua.UA_ERR_SHAPE
    assert _trace(good, rank=2) == ua.UA_ERR_RANK
    assert _trace(good, scale=0.0) == ua.UA_ERR_UNSUPPORTED
    assert _trace((0, 64, 4, 64), q=0, k=0, v=0, out=0, trace=0) == ua.UA_OK
    assert _store_only(good, out=0) == ua.UA_ERR_NULL
    assert _store_only(good, out=O + 2) == ua.UA_ERR_ALIGN
    assert _store_only((1, 64, 5, 64)) == ua.UA_ERR_SHAPE
    assert _store_only(good, rank=-1) == ua.UA_ERR_RANK
    assert _store_only((1, 64, 4, 96)) == ua.UA_ERR_UNSUPPORTED
    assert _store_only((2, 0, 4, 64), out=0) == ua.UA_OK


def test_work_units():
    # 256-row units when that gives at least 128 of them, else 128-row units;
    # d = 64 takes 512-row units (two row blocks per wave) when there are at
    # least 128 of them and the rounds over 256 CUs do not make it slower
    assert ua.work_units(1, 65536, 40, 128, 8) == 5 * 256
    assert ua.work_units(2, 32768, 24, 64, 4) == 2 * 6 * 64
    assert ua.work_units(2, 1100, 64, 64, 2) == 2 * 32 * 3
    assert ua.work_units(2, 16384, 24, 64, 4) == 2 * 6 * 64    # 384 units of 512 rows = 1.5 rounds
    assert ua.work_units(1, 4096, 48, 64, 2) == 24 * 8        # 24*8 >= 128 -> 512-row units
    assert ua.work_units(1, 4096, 24, 64, 2) == 12 * 16       # 12*8 < 128 -> 256-row units
    assert ua.work_units(1, 16384, 24, 128, 8) == 3 * 64
    assert ua.work_units(1, 4096, 24, 128, 8) == 3 * 32      # 3*16 < 128 -> 128-row units
    assert ua.work_units(1, 512, 4, 64, 2) == 2 * 4
    assert ua.work_units(3, 129, 9, 64, 3) == 3 * 3 * 2
    assert ua.work_units(0, 64, 4, 64, 2) == 0
    assert ua.work_units(1, 63, 4, 64, 2) == 0                 # invalid shape


def test_key_split_choice_and_workspace_size():
    # The rule: for launches with fewer than 1024 query tiles, the
    # plain call's shape (and, where that uses 128-row units, the 256-row one
    # on 64-key tiles) with n in 1..4 workgroups per tile, costing
    # rounds(n * tiles / 256) * (keys one wave processes + 512 + 128 (n - 1));
    # parts of at least 8 units of KS tiles.
    # video_dit (1280 tiles), mixed (3 full rounds) and tiny (too short): no split
    assert ua.key_split(1, 65536, 40, 128, 8) == 1 and ua.workspace_bytes(1, 65536, 40, 128, 8) == 0
    assert ua.key_split(2, 32768, 24, 64, 4) == 1 and ua.workspace_bytes(2, 32768, 24, 64, 4) == 0
    assert ua.key_split(1, 512, 4, 64, 2) == 1 and ua.workspace_bytes(1, 512, 4, 64, 2) == 0
    nx = 4 * 16 + 2                                 # floats per lane at d = 128: O^T blocks, m, l
    # dit_long: 192 tiles of 256 rows over 256 key tiles of 64.  The best
    # plain key split, n = 4 (768 workgroups = 3 rounds of 64 tiles: 3 *
    # (4096 + 512 + 384) = 14976), loses to stream-K: 256 workgroups of
    # 49152 / 256 = 192 iterations, L * 64 + 2 * 512 + 128 * (2 - 1) = 13440,
    # every query tile cut into at most 2 parts
    assert ua.key_split(1, 16384, 24, 128, 8) == 2 and ua.stream_k_iters(1, 16384, 24, 128, 8) == 192
    assert ua.workspace_bytes(1, 16384, 24, 128, 8) == 4096 + 192 * 2 * 8 * nx * 64 * 4
    # dit_image: 96 tiles of 128 rows (two key groups of 4 waves on 32-key
    # tiles): n = 2 (1024 + 640) beats n = 1 (2048 + 512), and the 256-row
    # shape on 64-key tiles split 4 ways (1024 + 896)
    assert ua.key_split(1, 4096, 24, 128, 8) == 2
    assert ua.workspace_bytes(1, 4096, 24, 128, 8) == 4096 + 96 * 2 * 4 * nx * 64 * 4
    assert ua.workspace_count_bytes(1, 4096, 24, 128, 8) == 4096   # counts of up to 1024 query tiles
    assert ua.workspace_count_bytes(1, 16384, 24, 128, 8) == 4096
    assert ua.workspace_count_bytes(1, 65536, 40, 128, 8) == 0
    # d = 64 with two row blocks per wave (nx = 2 * (2 * 16) + 4), 192 tiles
    assert ua.work_units(1, 16384, 48, 64, 8) == 6 * 32 and ua.key_split(1, 16384, 48, 64, 8) == 4
    assert ua.workspace_bytes(1, 16384, 48, 64, 8) == 4096 + 192 * 4 * 8 * 68 * 64 * 4
    # 160 tiles over 128 key tiles: n = 3 (480 workgroups, 2 rounds of 43
    # tiles: 2 * (2752 + 768)) beats n = 4 (3 rounds) and n = 1; the parts
    # are 42, 43, 43
    assert ua.key_split(1, 8192, 40, 64, 8) == 3
    # one head of 4096 keys: 32 tiles of 128 rows split 4 ways, 16 pairs of
    # 32-key tiles per workgroup (4 storing waves per workgroup)
    assert ua.key_split(1, 4096, 8, 128, 8) == 4
    assert ua.workspace_bytes(1, 4096, 8, 128, 8) == 4096 + 32 * 4 * 4 * nx * 64 * 4
    # 320 tiles (1.25 rounds) of video_dit's heads at 16384 keys: the best
    # plain split, n = 4 (five full rounds of 64 key tiles, 5 * 4992 = 24960),
    # loses to stream-K (320 iterations per workgroup: 20480 + 1024 + 128);
    # at 32768 keys 640 tiles (2.5 rounds) split 2 ways (five full rounds),
    # which stream-K does not beat by the 3% it must
    assert ua.key_split(1, 16384, 40, 128, 8) == 2 and ua.stream_k_iters(1, 16384, 40, 128, 8) == 320
    assert ua.workspace_bytes(1, 16384, 40, 128, 8) == 4096 + 320 * 2 * 8 * nx * 64 * 4
    assert ua.key_split(1, 32768, 40, 128, 8) == 2 and ua.stream_k_iters(1, 32768, 40, 128, 8) == 0
    assert ua.workspace_bytes(1, 32768, 40, 128, 8) == 4096 + 640 * 2 * 8 * nx * 64 * 4
    # an odd 32-key tile count puts the plain call on one wave per SIMD (4-wave
    # workgroups of 128 rows); the split runs the 8-wave 256-row shape instead:
    # 16 tiles split 4 ways over 64 key tiles (the last one half full)
    assert ua.key_split(1, 127 * 32, 8, 128, 8) == 4
    assert ua.workspace_bytes(1, 127 * 32, 8, 128, 8) == 4096 + 16 * 4 * 8 * nx * 64 * 4
    assert ua.key_split(0, 64, 4, 64, 2) == 0 and ua.key_split(1, 63, 4, 64, 2) == 0
    assert ua.workspace_bytes(1, 63, 4, 64, 2) == 0


def test_workspace_validation():
    shape = (1, 16384, 24, 128)                   # needs a workspace at P = 8
    need = ua.workspace_bytes(*shape, 8)
    for call in (_fused_ws, _serial_ws, _fused_io_ws):
        assert call(shape, P=8, ws=0) == ua.UA_ERR_NULL
        assert call(shape, P=8, ws=W + 8) == ua.UA_ERR_ALIGN
        assert call(shape, P=8, ws_bytes=need - 1) == ua.UA_ERR_WORKSPACE
        assert call(shape, P=8, ws_bytes=0) == ua.UA_ERR_WORKSPACE
        # the other arguments are checked first
        assert call(shape, P=8, q=0, ws=0) == ua.UA_ERR_NULL
        assert call(shape, P=8, rank=8, ws_bytes=0) == ua.UA_ERR_RANK
        assert call(shape, P=8, out=O + 2, ws_bytes=0) == ua.UA_ERR_ALIGN
        # empty calls need nothing
        assert call((0, 16384, 24, 128), P=8, q=0, k=0, v=0, out=0, ws=0, ws_bytes=0) == ua.UA_OK


def test_noalloc_validates_and_rejects_splits_beyond_its_scratch():
    L = ua.lib()

    def call(shape, rank=0, P=8, q=A, k=B_, v=C, out=O, scale=0.125):
        return L.attn_ulysses_fused_noalloc(q, k, v, rank, P, out, ctypes.byref(Shape(*shape)), scale, None)

    assert call((1, 4096, 24, 128), rank=8) == ua.UA_ERR_RANK
    assert call((1, 4096, 24, 96)) == ua.UA_ERR_UNSUPPORTED
    assert call((1, 4096, 24, 128), q=0) == ua.UA_ERR_NULL
    assert call((1, 4096, 24, 128), out=O + 2) == ua.UA_ERR_ALIGN
    assert call((0, 4096, 24, 128), q=0, k=0, v=0, out=0) == ua.UA_OK    # empty: nothing touched
    # the heads of the video workload at 32768 keys (640 query tiles split
    # 2 ways): ~165 MiB of partials, beyond the 128 MiB scratch
    need = ua.workspace_bytes(1, 32768, 40, 128, 8)
    assert need > ua.SCRATCH_BYTES == 128 << 20
    assert call((1, 32768, 40, 128)) == ua.UA_ERR_SCRATCH
    assert "scratch" in ua.status_string(ua.UA_ERR_SCRATCH)
    text = open(HEADER).read()
    assert re.search(r"#define\s+UA_SCRATCH_BYTES\s+\(\(size_t\)128 << 20\)", text)


def test_write_counts_validates_its_counter_buffer():
    L = ua.lib()

    def call(shape=(1, 4096, 24, 128), rank=0, P=8, counts=O + 4096, out=O, q=A, ws=None, ws_bytes=0):
        return L.ua_fused_write_counts(q, B_, C, rank, P, out, ctypes.byref(Shape(*shape)), ctypes.c_float(0.125),
                                       ws, ctypes.c_size_t(ws_bytes), None, counts)

    assert call(counts=0) == ua.UA_ERR_NULL
    assert call(counts=O + 4100) == ua.UA_ERR_ALIGN
    assert call(q=0) == ua.UA_ERR_NULL
    assert call(rank=8) == ua.UA_ERR_RANK
    assert call((1, 4096, 24, 96)) == ua.UA_ERR_UNSUPPORTED
    # a shape whose plan splits keys needs its workspace
    assert ua.key_split(1, 16384, 40, 128, 8) > 1
    assert call((1, 16384, 40, 128)) == ua.UA_ERR_NULL
    assert call((1, 16384, 40, 128), ws=A + 8192, ws_bytes=64) == ua.UA_ERR_WORKSPACE


def test_traced_workspace_call_validates_and_counts_its_workgroups():
    L = ua.lib()
    L.attn_ulysses_fused_trace_ws.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_void_p, ctypes.c_float,
                                                                       ctypes.c_void_p, ctypes.c_size_t,
                                                                       ctypes.c_void_p, ctypes.c_void_p]

    def call(shape=(1, 16384, 40, 128), rank=0, P=8, trace=O + 4096, out=O, ws=A + 8192, ws_bytes=1 << 30):
        return L.attn_ulysses_fused_trace_ws(A, B_, C, rank, P, out, ctypes.byref(Shape(*shape)), 0.125,
                                             ws, ws_bytes, None, trace)

    assert call(trace=0) == ua.UA_ERR_NULL
    assert call(trace=O + 4100) == ua.UA_ERR_ALIGN
    assert call(ws=0) == ua.UA_ERR_NULL                 # this shape splits: it needs the workspace
    assert call(ws_bytes=64) == ua.UA_ERR_WORKSPACE
    # workgroups of the split launch: the stream-K runs (one per CU), more
    # than the query tiles of the plain launch; equal otherwise
    for shape in ((1, 16384, 24, 128), (1, 16384, 40, 128), (1, 4096, 24, 128)):
        plain, split = ua.work_units(*shape, 8), ua.work_units(*shape, 8, workspace=True)
        if ua.key_split(*shape, 8) > 1:
            if ua.stream_k_iters(*shape, 8):
                B, S, H, d = shape
                total = plain * -(-S // 64)
                assert split == -(-total // ua.stream_k_iters(*shape, 8))
            else:
                assert split == plain * ua.key_split(*shape, 8)
        else:
            assert split == plain
    assert ua.work_units(1, 512, 4, 64, 2, workspace=True) == ua.work_units(1, 512, 4, 64, 2)


def test_tile_override_from_the_environment():
    """UA_TILE forces the launch shape (read once per process, so each
    setting runs in a fresh interpreter); unknown values and shapes it does
    not fit are ignored."""
    import subprocess
    import sys
    code = ("import comm_fusion_amd as ua; print(ua.work_units(2, 32768, 24, 64, 4), "
            "ua.work_units(1, 65536, 40, 128, 8), ua.work_units(1, 4064, 8, 128, 8), "
            "ua.key_split(1, 4096, 24, 128, 8))")

    def run(tile):
        env = dict(os.environ)
        env.pop("UA_TILE", None)
        if tile is not None:
            env["UA_TILE"] = tile
        out = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True,
                             check=True, timeout=300).stdout
        return tuple(int(x) for x in out.split())

    default = run(None)
    assert default == (768, 1280, 32, 2)          # mixed 512-row units, video 256, 4064 keys 128-row
    assert run("256x64") == (1536, 1280, 16, 4)   # 256-row units everywhere
    assert run("512x32") == (768, 1280, 32, 2)    # d = 64 only: the d = 128 shapes keep their choice
    assert run("128x64")[:3] == (3072, 2560, 32)  # 4-wave 128-row units
    assert run("128x32")[2] == 32                 # 127 key tiles of 32: odd, so ignored there
    assert run("nonsense") == default
