"""Small test-side helpers: bf16 bit-pattern conversions done with numpy."""
import numpy as np


def to_bf16(a) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def from_bf16(a) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(a) -> np.ndarray:
    """Round float values to the nearest bf16 value, returned as float32."""
    return from_bf16(to_bf16(a))


def rand_bf16(rng, shape, std=1.0) -> np.ndarray:
    return to_bf16(rng.standard_normal(shape) * std)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
