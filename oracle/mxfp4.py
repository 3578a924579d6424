"""MXFP4 weights for the oracle: OCP microscaling FP4 - E2M1 elements in blocks of 32 that share one
E8M0 (power-of-two) scale.

Test infrastructure only (see the package docstring for who may import it).

The pages name FP8/FP4 megakernels as their next step (P3 "Limitations and Future Plans"); as for
FP8, the model is unchanged and its matrices are stored quantized, so a step computes the same
layers over the dequantized weights w = value(code) * 2^(scale - 127).

E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no infinities or NaN. Exponent field 0
holds 0 and the subnormal 0.5; otherwise (1 + m/2) * 2^(e - 1). E8M0: an unsigned biased exponent,
value 2^(c - 127); code 255 is NaN.

Packed matrix layout (the boundary's too): a matrix of R rows and K inputs (K a multiple of 32) is
R rows of roundup16(K/2 + K/32) bytes - the K/2 code bytes (element 2i in the low nibble of byte i,
element 2i + 1 in the high nibble), then the K/32 block scales, then zero bytes up to a multiple of
16. Rows are held in ``Mxfp4Rows`` arrays, which remember K.
"""

import numpy as np


def row_bytes(k):
    return (k // 2 + k // 32 + 15) // 16 * 16


def k_of_row_bytes(nbytes):
    """The K (a multiple of 32) whose packed row is ``nbytes`` long. It is unique: K/32 * 17 bytes of
    codes and scales step by 17, more than the 16 bytes of padding."""
    for k in range(32, 32 * (nbytes // 17 + 2), 32):
        if row_bytes(k) == nbytes:
            return k
    raise ValueError(f"no MXFP4 row is {nbytes} bytes long")


def e2m1_table():
    """float64 value of each of the 16 codes, from the definition above."""
    out = np.empty(16, np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        out[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return out


_E2M1 = e2m1_table()


def e8m0_to_f64(codes):
    c = np.asarray(codes, np.int64)
    return np.where(c == 255, np.nan, np.exp2(c.astype(np.float64) - 127.0))


class Mxfp4Rows(np.ndarray):
    """Packed MXFP4 rows (uint8, last axis roundup16(K/2 + K/32)) that remember K."""

    def __new__(cls, data, k):
        obj = np.asarray(data, np.uint8).view(cls)
        obj.k = int(k)
        return obj

    def __array_finalize__(self, obj):
        self.k = getattr(obj, "k", None)

    def __reduce__(self):                     # (deepcopy / pickle keep K)
        fn, args, state = super().__reduce__()
        return fn, args, (state, self.k)

    def __setstate__(self, st):
        super().__setstate__(st[0])
        self.k = st[1]


def pack_rows(codes, scales):
    """codes [..., K] (0..15) and scales [..., K/32] (E8M0 bytes) -> Mxfp4Rows [..., row_bytes(K)]."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    k = codes.shape[-1]
    assert k % 32 == 0 and scales.shape[-1] == k // 32
    out = np.zeros(codes.shape[:-1] + (row_bytes(k),), np.uint8)
    out[..., : k // 2] = (codes[..., 0::2] & 0xF) | ((codes[..., 1::2] & 0xF) << 4)
    out[..., k // 2: k // 2 + k // 32] = scales
    return Mxfp4Rows(out, k)


def dequant_rows(packed, dtype=np.float32):
    """Mxfp4Rows [..., row_bytes(K)] -> [..., K] in dtype: value(code) * block scale, formed in
    float64 (exact) and then cast."""
    k = packed.k
    raw = np.asarray(packed, np.uint8)
    b = raw[..., : k // 2]
    codes = np.empty(raw.shape[:-1] + (k,), np.uint8)
    codes[..., 0::2] = b & 0xF
    codes[..., 1::2] = b >> 4
    scales = e8m0_to_f64(raw[..., k // 2: k // 2 + k // 32])
    vals = _E2M1[codes] * np.repeat(scales, 32, axis=-1)
    return vals.astype(dtype)
