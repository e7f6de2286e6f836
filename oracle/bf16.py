"""float64 -> bfloat16 rounding, round to nearest even.  (Oracle: test infrastructure only.)

Used to compare a bf16 GPU result against the exact (fp64) value rounded once
to bf16.  bfloat16 keeps float32's 8 exponent bits and 7 fraction bits; the
rounding is done from the float64 bits directly (no float32 detour, which
could round twice).  Zero, normal numbers in bf16's range only.
"""
from __future__ import annotations

import numpy as np


def f64_to_bf16_bits(x) -> np.ndarray:
    x = np.asarray(x, np.float64)
    u = x.view(np.uint64)
    sign = (u >> np.uint64(63)) & np.uint64(1)
    expo = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    frac = u & np.uint64((1 << 52) - 1)
    shift = np.uint64(45)
    keep = (frac >> shift).astype(np.int64)
    rem = frac & np.uint64((1 << 45) - 1)
    half = np.uint64(1 << 44)
    up = (rem > half) | ((rem == half) & ((keep & 1) == 1))
    keep = keep + up.astype(np.int64)
    expo = expo + (keep >> 7)
    keep = keep & 0x7F
    e8 = expo - 1023 + 127
    zero = (u & np.uint64((1 << 63) - 1)) == 0
    if np.any(~zero & ((e8 < 1) | (e8 > 254))):
        raise ValueError("value outside bf16 normal range")
    bits = (sign.astype(np.int64) << 15) | (np.where(zero, 0, e8) << 7) | np.where(zero, 0, keep)
    return bits.astype(np.uint16)
