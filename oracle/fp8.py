"""FP8 weights for the oracle: OCP E4M3 ("e4m3fn") codes with one float32 scale per matrix row.

Test infrastructure only (see the package docstring for who may import it).

The pages name FP8/FP4 megakernels as their next step (P3 "Limitations and Future Plans"); this
build's FP8 variant keeps the model and quantizes its matrices, so what a step computes with FP8
weights is the same step over the dequantized weights w = decode(code) * row_scale.

E4M3 (OCP 8-bit floating point, the variant without infinities): 1 sign bit, 4 exponent bits
(bias 7), 3 mantissa bits. Exponent field 0 holds the subnormals m/8 * 2^-6; codes S.1111.111 are
NaN; every other code is (1 + m/8) * 2^(e - 7). Largest finite value 448, smallest subnormal 2^-9.

Packed matrix layout (the boundary's too): a matrix of R rows and K inputs is R rows of K + 16
bytes - the K codes of the row, then the row's float32 scale (little-endian) and 12 zero bytes, so
that every row starts on a 16-byte boundary.
"""

import numpy as np

SCALE_BYTES = 16


def e4m3_table():
    """float64 value of each of the 256 codes, from the definition above."""
    out = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_TABLE = e4m3_table()


def e4m3_to_f64(codes):
    return _TABLE[np.asarray(codes, np.uint8)]


def is_packed(a):
    """Packed FP8 rows are uint8 arrays; bf16 matrices are uint16 arrays."""
    return np.asarray(a).dtype == np.uint8


def dequant_rows(packed, dtype=np.float32):
    """Packed rows [..., K + 16] uint8 -> dequantized matrix [..., K] in dtype: code * row scale,
    formed in float64 (exact: a 4-bit significand times a float32) and then cast."""
    packed = np.asarray(packed, np.uint8)
    k = packed.shape[-1] - SCALE_BYTES
    codes = packed[..., :k]
    scale = np.ascontiguousarray(packed[..., k:k + 4]).view(np.float32)[..., 0].astype(np.float64)
    return (e4m3_to_f64(codes) * scale[..., None]).astype(dtype)


def pack_rows(codes, scales):
    """codes [..., K] uint8 and scales [...] float32 -> packed rows [..., K + 16] uint8."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.float32)
    out = np.zeros(codes.shape[:-1] + (codes.shape[-1] + SCALE_BYTES,), np.uint8)
    out[..., :codes.shape[-1]] = codes
    out[..., codes.shape[-1]:codes.shape[-1] + 4] = scales[..., None].view(np.uint8).reshape(scales.shape + (4,))
    return out
