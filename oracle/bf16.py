"""bfloat16 bit patterns <-> float64, for the oracle.  Test infrastructure only.

bf16 is the upper half of an IEEE float32, so widening is exact: shift the 16
bits into the high half of a 32-bit word and reinterpret.
"""

import numpy as np


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of uint16 bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest bf16 (ties to even), returning uint16 bits.

    Goes through float32 first (float64 -> float32 is itself round-to-nearest-even);
    used only for reporting, never to produce a value the HIP path is compared with.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    r[nan] = np.uint16(0x7FC0)
    return r
