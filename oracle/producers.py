"""The producers either side of the decode: query quantisation and the paged
KV-cache write.

Test infrastructure only (see ``oracle/__init__``).

[T5] ``quantize_q_fp8``: the fp8 query is quantised per (sequence, kv head):
the scale is the largest |q| over that sequence's q_len tokens, the h_r query
heads of the kv head and the head dimension (at least 1e-6), divided by the
e4m3 maximum 448; the codes are the e4m3fn cast of q / descale (round to
nearest, ties to even), in fp32 throughout. [T5] module docstring ("Inputs
follow vLLM's paged KV cache") and the harness's KV pool: K and V are stored
as e4m3 codes of x / descale with one fp32 descale per (sequence, kv head);
the page names the KV-cache write as one of the kernels that run before the
decode but prints none.

Readings (where the pages are silent): the write puts the n_new newest tokens
of sequence b at positions L_b - n_new .. L_b - 1 (L_b = seq_lens[b], new
tokens included), row pos % page_size of page block_table[b][pos /
page_size], skipping a token whose position is negative or whose block-table
entry is missing or outside the pool; the descales are inputs; a value beyond the e4m3 range saturates
to +-448 and NaN stays NaN (0x7F). The latent-record write computes one scale
per token and 128-value block, the smallest power of two at or above the
block's largest |x| (at least 1e-6) over 448 in fp32 ("vLLM PR #62633",
Kernel design: the kernel dequantises a record exactly to bf16, which a code
times an arbitrary fp32 scale would not allow: the code carries 4 significant
bits and bf16 8), stores the codes of x / scale, copies the 64 bf16 rope
values bitwise and stores the four fp32 scales.

Pinned by tests/test_producers_oracle.py: encode_e4m3 against torch's
float8_e4m3fn cast over a dense sweep of the finite range, the round trip of
every finite code, ties to even, saturation and NaN; quantize_q on a
hand-worked example and its invariants (the largest |q| of a group maps to
+-448, a zero group gives zero codes); the writes by hand-worked positions and
by the error bound of the round trip.
"""

import math

import numpy as np

from .formats import E4M3_TABLE

E4M3_MAX = 448.0

# finite non-negative codes 0x00 .. 0x7E in increasing value
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = E4M3_TABLE[:0x7F]


def encode_e4m3(x) -> np.ndarray:
    """float32 values -> e4m3fn codes: round to the nearest representable
    value, ties to the even code, |x| beyond 448 saturates to +-448, NaN gives
    0x7F; the sign of -0.0 is kept."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    a = np.where(np.isnan(a), 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    codes = np.where(np.signbit(x), mag | 0x80, mag).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), codes).astype(np.uint8)


def quantize_q(q, num_seqs, q_len, h_k):
    """q: float32 [num_seqs * q_len, h_q, d] (widened bf16) -> (codes uint8
    same shape, q_descale float32 [num_seqs, h_k])."""
    q = np.asarray(q, dtype=np.float32)
    _, h_q, d = q.shape
    h_r = h_q // h_k
    qg = q.reshape(num_seqs, q_len, h_k, h_r, d)
    amax = np.abs(qg).max(axis=(1, 3, 4)).astype(np.float32)
    amax = np.maximum(amax, np.float32(1e-6))
    descale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    y = (qg / descale[:, None, :, None, None]).astype(np.float32)
    return encode_e4m3(y).reshape(q.shape), descale


def write_positions(seq_lens, n_new, block_table, page_size, num_pages=None):
    """(page, row) of each new token, [num_seqs, n_new] each; page -1 marks a
    token with no slot (position < 0, past the block table, or an entry outside
    [0, num_pages)), which the write skips."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    bt = np.asarray(block_table)
    pos = lens[:, None] - n_new + np.arange(n_new)[None, :]
    blk = pos // page_size
    ok = (pos >= 0) & (blk < bt.shape[1])
    pages = np.take_along_axis(bt, np.where(ok, blk, 0), axis=1).astype(np.int64)
    if num_pages is not None:
        ok &= (pages >= 0) & (pages < num_pages)
    return np.where(ok, pages, -1), np.where(ok, pos % page_size, 0)


def write_kv_e4m3(cache, x_new, seq_lens, n_new, block_table, descale):
    """Return a copy of `cache` (uint8 [pages, page_size, h_k, d]) with the new
    tokens x_new (float32 [num_seqs * n_new, h_k, d]) written as
    e4m3(x / descale[b, g])."""
    out = np.array(cache, copy=True)
    page_size = out.shape[1]
    num_seqs = len(seq_lens)
    x = np.asarray(x_new, dtype=np.float32).reshape(num_seqs, n_new, *out.shape[2:])
    ds = np.asarray(descale, dtype=np.float32)
    pages, rows = write_positions(seq_lens, n_new, block_table, page_size, out.shape[0])
    for b in range(num_seqs):
        for t in range(n_new):
            if pages[b, t] < 0:
                continue
            y = (x[b, t] / ds[b][:, None]).astype(np.float32)
            out[pages[b, t], rows[b, t]] = encode_e4m3(y)
    return out


def pow2_ceil(v):
    """The smallest power of two >= v > 0 (v = m 2^e with m in [0.5, 1): v
    itself when m = 0.5, else 2^e)."""
    m, e = math.frexp(float(v))
    return float(v) if m == 0.5 else math.ldexp(1.0, e)


def write_kv_latent(lat, rope, scl, x_new, rope_new, seq_lens, n_new, block_table):
    """Latent-record write. lat uint8 [pages, ps, 512], rope uint16 [pages, ps,
    64] (bf16 bits), scl float32 [pages, ps, 4]; x_new float32 [num_seqs *
    n_new, 512], rope_new uint16 [num_seqs * n_new, 64]. Returns the three
    updated copies."""
    lat, rope, scl = np.array(lat, copy=True), np.array(rope, copy=True), np.array(scl, copy=True)
    page_size = lat.shape[1]
    num_seqs = len(seq_lens)
    x = np.asarray(x_new, dtype=np.float32).reshape(num_seqs, n_new, 4, 128)
    r = np.asarray(rope_new, dtype=np.uint16).reshape(num_seqs, n_new, -1)
    pages, rows = write_positions(seq_lens, n_new, block_table, page_size, lat.shape[0])
    for b in range(num_seqs):
        for t in range(n_new):
            if pages[b, t] < 0:
                continue
            amax = np.maximum(np.abs(x[b, t]).max(axis=1).astype(np.float32), np.float32(1e-6))
            s = np.array([pow2_ceil(v) for v in (amax / np.float32(E4M3_MAX)).astype(np.float32)], np.float32)
            lat[pages[b, t], rows[b, t]] = encode_e4m3((x[b, t] / s[:, None]).astype(np.float32)).reshape(-1)
            scl[pages[b, t], rows[b, t]] = s
            rope[pages[b, t], rows[b, t]] = r[b, t]
    return lat, rope, scl


def nvfp4_kernel_values(packed, scales):
    """NVFP4 K/V rows -> the values the decode multiplies ([T5] KV cache
    formats and ``nvfp4_quantize``): packed e2m1 codes (..., d/2) with one
    e4m3 scale byte per 16 elements (..., d/16); value = e4m3(code * scale *
    2^-3), rounded to nearest, ties to even (the product is exact in float32:
    at most 6 significant bits). The host folds the 2^3 back into the
    descale."""
    from .formats import E2M1_TABLE, E4M3_TABLE, unpack_fp4

    codes = E2M1_TABLE[unpack_fp4(np.asarray(packed))]
    sc = np.repeat(E4M3_TABLE[np.asarray(scales)], 16, axis=-1)
    prod = (codes * sc * 0.125).astype(np.float32)
    assert np.array_equal(prod.astype(np.float64), codes * sc * 0.125)  # exact
    return E4M3_TABLE[encode_e4m3(prod)]
