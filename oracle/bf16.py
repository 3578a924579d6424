"""bfloat16 codec for the oracle (test infrastructure only).

Weights and the KV cache are stored in BF16 (P1 "Decode is a bandwidth game"; P2 body). A bf16
value is the upper 16 bits of an IEEE binary32, so decoding is exact: shift the 16-bit pattern into
the top half of a 32-bit word. Encoding rounds to nearest, ties to even (the usual bf16 rounding).
"""

import numpy as np


def bf16_to_f32(u16):
    """Decode bf16 bit patterns (uint16 array) to float32, exactly."""
    u = np.asarray(u16, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """Round float32 values to bf16 bit patterns (round to nearest, ties to even).

    NaN inputs give a quiet NaN pattern with the sign kept; infinities pass through."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32)
    nan = np.isnan(x)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits.astype(np.uint64) + np.uint64(0x7FFF) + lsb.astype(np.uint64)) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    if nan.any():
        out = np.where(nan, ((bits >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16), out)
    return out


def f64_to_bf16(x):
    """Round float64 values straight to bf16 (nearest, ties to even), without a float32 detour.

    Used by the fp64 variant of the oracle so that its KV-cache writes are rounded once. Normal
    numbers only (values whose magnitude is at least 2**-126); the workloads never produce others.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    q = np.rint(np.ldexp(m, 8))             # 8 significant bits, rint = ties to even
    y = np.ldexp(q, e - 8)                  # exactly representable in bf16 (and float32)
    return (y.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
