"""Element formats read by the decode path: OCP e4m3 (fp8), bf16, and the
packed 4-bit e2m1 (fp4) KV format.

Test infrastructure only (see ``oracle/__init__``).

[T5] module docstring and ``quantize_q_fp8``: the KV cache and the fp8 query
are ``float8_e4m3fn`` (the OCP 8-bit E4M3 format: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, a single NaN mantissa pattern,
largest finite value 448). The page's harness poisons unused pages with the
byte 0x7F and calls it the e4m3fn NaN; it names 448 as the e4m3 maximum.

The narrow KV formats of [T5] (module docstring "KV cache formats" and
"Narrow KV formats: value tables, quantization and bit packing"): e2m1 has
1 sign bit, 2 exponent bits with bias 1 and 1 mantissa bit, no infinities
and no NaN; exponent 0 is subnormal (m/2 * 2^(1-bias)). A row of d codes is
stored as a little-endian bitstream of d/2 bytes: element 2i in the low
nibble of byte i, element 2i+1 in its high nibble.

Pinned by tests/test_oracle.py: known codes (0x7E = 448, 0x08 = 2^-6,
0x01 = 2^-9, 0x38 = 1, 0x7F/0xFF = NaN, sign symmetry), strict monotonicity
of the finite positive codes, and agreement with torch's float8_e4m3fn cast;
the e2m1 value set (golden file of the OCP MX fp4 values), the nibble order
on hand-packed bytes, and the packed decode against a bit-field decode in
``oracle.brute``.
"""

import numpy as np


def _e4m3_value(code: int) -> float:
    """Value of one e4m3fn byte, straight from the format definition."""
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:  # subnormal: 2^(1 - bias) * (m / 8)
        return sign * (2.0 ** (1 - 7)) * (man / 8.0)
    return sign * (2.0 ** (exp - 7)) * (1.0 + man / 8.0)


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_TABLE.setflags(write=False)


def decode_e4m3(codes) -> np.ndarray:
    """uint8 e4m3fn codes (any shape, any strides) -> float64 values."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"e4m3 codes must be uint8, got {c.dtype}")
    return E4M3_TABLE[c]


def decode_bf16(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 values (bf16 is the top half of an
    IEEE binary32, so widening the bits is exact)."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(f"bf16 bits must be uint16, got {b.dtype}")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _e2m1_value(code: int) -> float:
    """Value of one e2m1 code (4 bits), straight from the format definition."""
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:  # subnormal: 2^(1 - bias) * (m / 2)
        return sign * (man / 2.0)
    return sign * (2.0 ** (exp - 1)) * (1.0 + man / 2.0)


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_TABLE.setflags(write=False)


def unpack_fp4(packed) -> np.ndarray:
    """uint8 bytes (..., d/2) -> uint8 codes (..., d): element 2i is the low
    nibble of byte i, element 2i+1 its high nibble."""
    b = np.asarray(packed)
    if b.dtype != np.uint8:
        raise TypeError(f"packed fp4 rows must be uint8, got {b.dtype}")
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def decode_e2m1_packed(packed) -> np.ndarray:
    """Packed e2m1 rows (..., d/2) uint8 -> float64 values (..., d)."""
    return E2M1_TABLE[unpack_fp4(packed)]


KV_DECODERS = {"e4m3": decode_e4m3, "e2m1": decode_e2m1_packed}
