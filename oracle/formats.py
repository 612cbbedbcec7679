"""Element formats read by the decode path: OCP e4m3 (fp8) and bf16.

Test infrastructure only (see ``oracle/__init__``).

[T5] module docstring and ``quantize_q_fp8``: the KV cache and the fp8 query
are ``float8_e4m3fn`` (the OCP 8-bit E4M3 format: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, a single NaN mantissa pattern,
largest finite value 448). The page's harness poisons unused pages with the
byte 0x7F and calls it the e4m3fn NaN; it names 448 as the e4m3 maximum.

Pinned by tests/test_oracle.py: known codes (0x7E = 448, 0x08 = 2^-6,
0x01 = 2^-9, 0x38 = 1, 0x7F/0xFF = NaN, sign symmetry), strict monotonicity
of the finite positive codes, and agreement with torch's float8_e4m3fn cast.
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
