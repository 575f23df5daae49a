"""The Python binding rejects bad tensors before calling the library (CPU
only for what needs no GPU tensor; the size and layout checks that need
device tensors are in the GPU part below)."""
import pytest
import torch

import comm_fusion_amd as ua


def _t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def test_qkv_shapes_must_agree():
    with pytest.raises(ValueError):
        ua.attn_ulysses_fused(_t(1, 64, 2, 64), _t(1, 64, 2, 64), _t(1, 32, 2, 64), 0, 2, _t(16384))
    with pytest.raises(ValueError):
        ua.attn_serial(_t(64, 2, 64), _t(64, 2, 64), _t(64, 2, 64), 0, 2, _t(8192))


def test_host_or_non_bf16_tensors_are_rejected():
    q = _t(1, 64, 2, 64)
    with pytest.raises(TypeError):          # host tensors
        ua.attn_ulysses_fused(q, q, q, 0, 2, _t(16384))
    f = _t(1, 64, 2, 64, dtype=torch.float32)
    with pytest.raises(TypeError):          # not bfloat16
        ua.attn_serial(f, f, f, 0, 2, _t(1, 64, 2, 64))


def test_sequence_partitioned_inputs_must_match_p():
    x = _t(1, 4, 16, 8, 64)                 # [B][P=4][S/P][H][d]
    with pytest.raises(ValueError):
        ua.attn_ulysses_fused_io(x, x, x, 0, 2, _t(1 * 64 * 8 * 64))
    with pytest.raises(ValueError):
        ua.a2a_gather(x, 0, 2, _t(1, 64, 4, 64))
    with pytest.raises(ValueError):
        ua.a2a_gather(_t(64, 8, 64), 0, 2, _t(1, 64, 4, 64))
    with pytest.raises(ValueError):
        ua.a2a_permute(_t(64, 4, 64), 0, 2, _t(1 * 64 * 8 * 64))


@pytest.mark.gpu
def test_device_tensor_sizes_and_layouts_are_checked():
    d = torch.device("cuda:0")
    q = torch.zeros((1, 64, 2, 64), dtype=torch.bfloat16, device=d)
    with pytest.raises(ValueError):         # out one element short
        ua.attn_ulysses_fused(q, q, q, 0, 2, torch.zeros(64 * 4 * 64 - 1, dtype=torch.bfloat16, device=d))
    wide = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device=d)
    with pytest.raises(TypeError):          # a non-contiguous view
        ua.attn_serial(wide[:, :, :2], wide[:, :, :2], wide[:, :, :2], 0, 2, q.clone())
    x = torch.zeros((1, 64, 4, 64), dtype=torch.bfloat16, device=d)
    with pytest.raises(ValueError):         # X_local of the wrong size
        ua.a2a_gather(x, 0, 2, torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device=d))
    out = torch.zeros(64 * 4 * 64, dtype=torch.bfloat16, device=d)
    with pytest.raises(ua.UAError) as e:    # rank out of range reaches the C validation
        ua.attn_ulysses_fused(q, q, q, 2, 2, out)
    assert e.value.status == ua.UA_ERR_RANK


def test_tensors_of_one_call_must_share_a_device():
    # the device check runs before any stream or device is touched
    from types import SimpleNamespace
    from comm_fusion_amd import _binding
    a = SimpleNamespace(device=torch.device("cuda", 0))
    b = SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError):
        _binding._stream(None, a, b)
    s = SimpleNamespace(device=torch.device("cuda", 1), cuda_stream=1234)
    with pytest.raises(ValueError):
        _binding._stream(s, a, a)
    assert _binding._stream(s, b, b) == 1234
    assert _binding._stream(5678, a, a) == 5678      # a raw handle is taken as given


def test_library_shares_the_hip_runtime_that_torch_loads():
    # Loading the library through the binding before torch has been imported
    # must still leave one HIP runtime in the process (torch's): two copies
    # would make torch's pointers and streams invalid in the library's calls.
    import subprocess
    import sys
    code = ("import comm_fusion_amd as ua; ua.lib(); import torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print(len(paths)); print(paths)\n")
    root = __import__("os").path.dirname(__import__("os").path.dirname(__import__("os").path.abspath(__file__)))
    out = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    lines = out.stdout.strip().splitlines()
    assert lines[0] == "1", lines
