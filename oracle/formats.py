"""Element formats read by the decode path: OCP e4m3 (fp8), bf16, and the
packed narrow KV formats e2m1 (fp4), e2m3 and e3m2 (fp6).

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

The fp6 formats of the same list ([T5] "e2m3", "e3m2"; OCP MX FP6): e2m3 has
2 exponent bits with bias 1 and 3 mantissa bits (largest 7.5), e3m2 has 3
exponent bits with bias 3 and 2 mantissa bits (largest 28); both have 1 sign
bit, no infinities and no NaN, and exponent 0 is subnormal
(m/2^M * 2^(1-bias)). A row of d codes (d a multiple of 4) is a little-endian
bitstream of 3d/4 bytes ([T5] ``pack_subbyte``): element i occupies bits
6i .. 6i+5, so four codes fill three bytes.

Pinned by tests/test_oracle.py: known codes (0x7E = 448, 0x08 = 2^-6,
0x01 = 2^-9, 0x38 = 1, 0x7F/0xFF = NaN, sign symmetry), strict monotonicity
of the finite positive codes, and agreement with torch's float8_e4m3fn cast;
the e2m1 value set (golden file of the OCP MX fp4 values), the nibble order
on hand-packed bytes, and the packed decode against a bit-field decode in
``oracle.brute``; the e2m3 / e3m2 value sets (largest and smallest values,
counts, every value exact in e4m3 via torch's cast), a hand-packed fp6 row
(golden file), and the fp6 decode against the bit-field decode.
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


def _fp6_value(code: int, exp_bits: int) -> float:
    """Value of one 6-bit code with `exp_bits` exponent bits (2: e2m3, 3: e3m2)."""
    man_bits = 5 - exp_bits
    bias = (1 << (exp_bits - 1)) - 1
    sign = -1.0 if code & 0x20 else 1.0
    exp = (code >> man_bits) & ((1 << exp_bits) - 1)
    man = code & ((1 << man_bits) - 1)
    if exp == 0:  # subnormal: 2^(1 - bias) * (m / 2^M)
        return sign * (2.0 ** (1 - bias)) * (man / float(1 << man_bits))
    return sign * (2.0 ** (exp - bias)) * (1.0 + man / float(1 << man_bits))


E2M3_TABLE = np.array([_fp6_value(c, 2) for c in range(64)], dtype=np.float64)
E3M2_TABLE = np.array([_fp6_value(c, 3) for c in range(64)], dtype=np.float64)
E2M3_TABLE.setflags(write=False)
E3M2_TABLE.setflags(write=False)


def unpack_fp6(packed) -> np.ndarray:
    """uint8 bytes (..., 3d/4) -> uint8 codes (..., d): element i is bits
    6i .. 6i+5 of the row read as one little-endian number."""
    b = np.asarray(packed)
    if b.dtype != np.uint8:
        raise TypeError(f"packed fp6 rows must be uint8, got {b.dtype}")
    if b.shape[-1] % 3:
        raise ValueError("a packed fp6 row holds a multiple of 3 bytes")
    t = b.reshape(b.shape[:-1] + (b.shape[-1] // 3, 3)).astype(np.uint32)
    w = t[..., 0] | (t[..., 1] << 8) | (t[..., 2] << 16)  # 24 bits = 4 codes
    out = np.stack([(w >> (6 * j)) & 0x3F for j in range(4)], axis=-1)
    return out.reshape(b.shape[:-1] + (4 * (b.shape[-1] // 3),)).astype(np.uint8)


def decode_e2m3_packed(packed) -> np.ndarray:
    """Packed e2m3 rows (..., 3d/4) uint8 -> float64 values (..., d)."""
    return E2M3_TABLE[unpack_fp6(packed)]


def decode_e3m2_packed(packed) -> np.ndarray:
    """Packed e3m2 rows (..., 3d/4) uint8 -> float64 values (..., d)."""
    return E3M2_TABLE[unpack_fp6(packed)]


KV_DECODERS = {"e4m3": decode_e4m3, "e2m1": decode_e2m1_packed, "e2m3": decode_e2m3_packed,
               "e3m2": decode_e3m2_packed}
KV_BITS = {"e4m3": 8, "e2m1": 4, "e2m3": 6, "e3m2": 6}


def kv_row_elems(row_bytes: int, kv_format: str) -> int:
    """Elements in a stored K/V row of `row_bytes` bytes."""
    return row_bytes * 8 // KV_BITS[kv_format]
