"""Test utilities: moving seeded arrays to the GPU and the comparison rules.

Tolerances (stated once, used by every parity test):
  bf16 outputs:  |gpu - ref64| <= 2 * ulp_bf16(max(|ref64|, 2**-8 * rms(ref64)))
                 with ulp_bf16(x) = 2**(floor(log2 x) - 7).  The floor keeps
                 values that cancel to near zero from demanding more than fp32
                 can give; rms is over the whole compared tensor.
  fp32 outputs:  |gpu - ref64| <= 1e-5 * max(|ref64|, rms(ref64)).
  weight grads:  the same rules with the floor taken from that dimension's
                 sqrt(sum of squared terms) instead of the rms.
  bit-exact:     v, dv in the dqkv v slots, paged-store locations, untouched
                 memory (sentinels).
"""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda"


def gpu_available() -> bool:
    return torch.cuda.is_available() and torch.cuda.device_count() > 0


def to_dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Seeded host array (bf16 as uint16 bits, or fp32) -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    if dtype == "int32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)
    raise ValueError(dtype)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host array of its stored bits (uint16 for bf16, float32 for fp32)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.contiguous().cpu().numpy()
    raise ValueError(t.dtype)


def host_value(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> fp64 (exact)."""
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(bits, dtype=np.float32).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    return np.exp2(np.floor(np.log2(x)) - 7)


def assert_close(gpu_bits: np.ndarray, ref64: np.ndarray, dtype: str, what: str, scale=None,
                 ulps: float = 2.0) -> None:
    """Element-wise tolerance check of stored GPU results against the fp64 oracle (rules above).

    ``gpu_bits`` are stored values (bf16 bit patterns or fp32); ``scale`` is the
    magnitude the floor is taken from: the rms of ``ref64`` by default.
    """
    assert_values_close(host_value(gpu_bits, dtype), ref64, dtype, what, scale, ulps)


def max_ulps_bf16(got: np.ndarray, ref64: np.ndarray) -> float:
    """Largest |got - ref| in bf16 ulps of max(|ref|, 2**-8 * rms(ref)) (a report, not a check)."""
    ref = np.asarray(ref64, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    floor = 2.0 ** -8 * np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref) / ulp_bf16(np.maximum(np.maximum(np.abs(ref), floor), 1e-30))))


def assert_values_close(got: np.ndarray, ref64: np.ndarray, rule: str, what: str, scale=None,
                        ulps: float = 2.0) -> None:
    """Tolerance check of GPU values (already decoded) under the ``rule`` of a dtype.

    Used directly for the fp32 norm-weight grads, which follow the rule of the
    activation dtype with the floor taken from ``scale`` (per element).  ``ulps``
    widens the bf16 rule where a documented chain of library roundings precedes
    the compared value (the MLA drafter layer); it is 2 everywhere else.
    """
    ref = np.asarray(ref64, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    if ref.size == 0:
        return
    if scale is None:
        scale = np.sqrt(np.mean(ref * ref))
    if rule == "bf16":
        tol = ulps * ulp_bf16(np.maximum(np.maximum(np.abs(ref), 2.0 ** -8 * np.asarray(scale)), 1e-30))
    else:
        tol = 1e-5 * np.maximum(np.abs(ref), np.asarray(scale))
    tol = np.broadcast_to(tol, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.flatnonzero(bad.reshape(-1))
        ratio = (err / np.maximum(tol, 1e-300)).reshape(-1)
        j = i[np.argmax(ratio[i])]
        raise AssertionError(
            f"{what}: {i.size} of {ref.size} values out of tolerance; worst at flat index {j}: "
            f"gpu {got.reshape(-1)[j]!r} ref {ref.reshape(-1)[j]!r} tol {tol.reshape(-1)[j]!r}")


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str) -> None:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    if not np.array_equal(a.view(np.uint8), b.view(np.uint8)):
        ne = np.flatnonzero(a.reshape(-1).view(np.uint16 if a.dtype == np.uint16 else np.uint32)
                            != b.reshape(-1).view(np.uint16 if b.dtype == np.uint16 else np.uint32))
        raise AssertionError(f"{what}: {ne.size} values differ bitwise, first at {ne[:5]}")


def announce(case: str) -> None:
    """Name the case (flushed) before a GPU step, so a fault names what ran."""
    print(f"[gpu case] {case}", flush=True)
