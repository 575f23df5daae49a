"""Shared helpers for the GPU parity tests (bf16 bit transfer, sentinel, checks)."""
import numpy as np

from ua_inputs import SENTINEL_BITS

# Value tolerance against the fp64 oracle on bf16 outputs, over all compared
# elements: max-abs and mean-abs as stated for this path, plus a relative RMS
# guard (outputs shrink like 1/sqrt(S) at long sequences, where the absolute
# bounds alone would admit a large relative error).  Expected GPU error is
# about 2^-9 relative (bf16 rounding of the output and of P).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_RMS = 1e-2


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def to_host_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel_buffer(n: int):
    import torch
    return torch.full((n,), SENTINEL_BITS - 0x10000 if SENTINEL_BITS >= 0x8000 else SENTINEL_BITS,
                      dtype=torch.int16, device="cuda").view(torch.bfloat16)


def empty_bf16(n: int):
    import torch
    return torch.empty((n,), dtype=torch.bfloat16, device="cuda")


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def value_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "mean_abs": float(err.mean()) if err.size else 0.0,
        "rel_rms": float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300))) if err.size else 0.0,
    }


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    e = value_errors(got, ref)
    assert e["max_abs"] <= MAX_ABS and e["mean_abs"] <= MEAN_ABS and e["rel_rms"] <= REL_RMS, \
        "%s: %s" % (what, e)
    return e


def check_dest_layout(dest_bits: np.ndarray, B, S, H, d, P, rank):
    """Slots of other ranks' heads keep the sentinel bits; this rank's slots
    are all written (not the sentinel).  Uses the [B][S][H][d] identity."""
    Hl = H // P
    v = dest_bits.reshape(B, S, H, d)
    own = v[:, :, rank * Hl:(rank + 1) * Hl]
    others = np.delete(v, np.s_[rank * Hl:(rank + 1) * Hl], axis=2)
    assert np.all(others == SENTINEL_BITS), "a slot of another rank's head was written"
    n_sent = int(np.count_nonzero(own == SENTINEL_BITS))
    assert n_sent == 0, "%d owned elements still hold the sentinel" % n_sent
    return own
