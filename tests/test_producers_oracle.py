"""Pins of oracle/producers.py (query quantisation, paged KV-cache write).

encode_e4m3 is checked against torch's float8_e4m3fn cast (an independent
library routine) over the finite range; quantize_q against a hand-worked
example ([T5] quantize_q_fp8's rule worked by hand) and invariants; the writes
against hand-worked positions and the round-trip error bound.
"""

import numpy as np
import pytest
import torch

from oracle.formats import E4M3_TABLE, decode_e4m3
from oracle.producers import encode_e4m3, quantize_q, write_kv_e4m3, write_kv_latent, write_positions


def torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_dense_sweep():
    rng = np.random.default_rng(7)
    finite = E4M3_TABLE[np.isfinite(E4M3_TABLE)]
    mids = (np.sort(finite)[1:] + np.sort(finite)[:-1]) / 2  # exact ties
    sweep = np.concatenate([np.linspace(-448, 448, 200001), mids, rng.standard_normal(100000) * 50,
                            rng.standard_normal(100000) * 1e-3, finite]).astype(np.float32)
    sweep = sweep[np.abs(sweep) <= 448]
    assert np.array_equal(encode_e4m3(sweep), torch_e4m3(sweep))


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if np.isfinite(E4M3_TABLE[c])], dtype=np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes).astype(np.float32)), codes)


def test_ties_go_to_even_code():
    # 1.0 (0x38) and 1.125 (0x39): the midpoint 1.0625 goes to 0x38; 1.125/1.25 -> 1.1875 goes to 0x3A
    assert encode_e4m3(np.float32(1.0625)) == 0x38
    assert encode_e4m3(np.float32(1.1875)) == 0x3A
    # smallest subnormal 2^-9 (0x01): half of it ties to 0 (even), a bit more rounds up
    assert encode_e4m3(np.float32(2.0 ** -10)) == 0x00
    assert encode_e4m3(np.float32(2.0 ** -10 * 1.01)) == 0x01


def test_saturation_nan_and_sign():
    x = np.array([448, 449, 464, 1000, np.inf, -1000, -np.inf, np.nan, -0.0, 0.0], dtype=np.float32)
    assert encode_e4m3(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x80, 0x00]


def test_quantize_q_hand_worked():
    # one sequence, q_len 1, h_q 2 on h_k 1, d 2: amax 4 -> descale 4/448;
    # q/descale = 112, -224, 56, 448 -> 0x6E (2^6*1.75), 0xF6 (-2^7*1.75), 0x66 (2^5*1.75), 0x7E
    q = np.array([[[1.0, -2.0], [0.5, 4.0]]], dtype=np.float32)
    codes, ds = quantize_q(q, num_seqs=1, q_len=1, h_k=1)
    assert ds.tolist() == [[np.float32(4.0) / np.float32(448.0)]]
    assert codes.reshape(-1).tolist() == [0x6E, 0xF6, 0x66, 0x7E]


def test_quantize_q_invariants():
    rng = np.random.default_rng(3)
    num_seqs, q_len, h_k, h_r, d = 3, 4, 2, 8, 128
    q = (rng.standard_normal((num_seqs * q_len, h_k * h_r, d)) * rng.uniform(0.1, 10)).astype(np.float32)
    q[:q_len, :h_r] = 0.0  # (seq 0, head group 0) all zero
    codes, ds = quantize_q(q, num_seqs, q_len, h_k)
    vals = decode_e4m3(codes).reshape(num_seqs, q_len, h_k, h_r, d)
    amax = np.abs(vals).max(axis=(1, 3, 4))
    assert amax[0, 0] == 0 and ds[0, 0] == np.float32(1e-6) / np.float32(448)
    assert np.all(amax.reshape(-1)[1:] == 448)
    # round trip within half an e4m3 step (relative 2^-4) above the subnormal range
    rec = vals * ds[:, None, :, None, None]
    qg = q.reshape(vals.shape)
    big = np.abs(qg) > 2.0 ** -6 * ds[:, None, :, None, None]
    assert np.all(np.abs(rec - qg)[big] <= np.abs(qg)[big] * 2.0 ** -4 + 1e-30)


def test_write_positions_hand_worked():
    # seq 0: L=5, two new tokens at 3, 4 -> page bt[0][0] rows 3, 0 of page bt[0][1] (page_size 4)
    bt = np.array([[7, 2, 9], [1, 4, 5]])
    pages, rows = write_positions([5, 12], 2, bt, 4)
    assert pages.tolist() == [[7, 2], [5, 5]] and rows.tolist() == [[3, 0], [2, 3]]


def test_write_kv_e4m3_touches_only_new_rows():
    rng = np.random.default_rng(5)
    pages, ps, h_k, d, n_new = 6, 4, 2, 8, 3
    cache = rng.integers(0, 256, size=(pages, ps, h_k, d), dtype=np.uint8)
    bt = np.array([[3, 0, 5], [1, 2, 4]])
    lens = [6, 9]
    x = rng.standard_normal((2 * n_new, h_k, d)).astype(np.float32)
    ds = np.array([[0.01, 0.02], [0.005, 1.0]], dtype=np.float32)
    out = write_kv_e4m3(cache, x, lens, n_new, bt, ds)
    pg, rw = write_positions(lens, n_new, bt, ps)
    touched = np.zeros((pages, ps), bool)
    touched[pg.reshape(-1), rw.reshape(-1)] = True
    assert np.array_equal(out[~touched], cache[~touched])
    for b in range(2):
        for t in range(n_new):
            got = decode_e4m3(out[pg[b, t], rw[b, t]]) * ds[b][:, None]
            want = x[b * n_new + t]
            sat = np.minimum(np.abs(want), 448 * ds[b][:, None])
            assert np.all(np.abs(got - np.sign(want) * sat) <= sat * 2.0 ** -4 + ds[b][:, None] * 2.0 ** -10)


def test_write_kv_latent_scales_and_rope():
    rng = np.random.default_rng(9)
    pages, ps, n_new = 4, 8, 2
    lat = np.zeros((pages, ps, 512), np.uint8)
    rope = np.zeros((pages, ps, 64), np.uint16)
    scl = np.zeros((pages, ps, 4), np.float32)
    bt = np.array([[2, 0], [3, 1]])
    x = rng.standard_normal((2 * n_new, 512)).astype(np.float32)
    x[0, 128:256] = 0.0  # a zero block: 1e-6 / 448 = 2.23e-9 rounds up to the scale 2^-28, codes 0
    x[1, 0:128] = 0.0
    x[1, 5] = 300.0  # 300 / 448 = 0.67 -> scale 1; e4m3(300) = 288 (step 32 above 256)
    x[1, 128:256] = 0.0
    x[1, 130] = -448.0 * 2.0 ** -7  # 448 * 2^-7 / 448 is a power of two already: scale 2^-7, code -448
    rn = rng.integers(0, 65536, size=(2 * n_new, 64), dtype=np.uint16)
    lat2, rope2, scl2 = write_kv_latent(lat, rope, scl, x, rn, [3, 16], n_new, bt)
    pg, rw = write_positions([3, 16], n_new, bt, ps)
    for b in range(2):
        for t in range(n_new):
            i = b * n_new + t
            vals = decode_e4m3(lat2[pg[b, t], rw[b, t]]).reshape(4, 128)
            s = scl2[pg[b, t], rw[b, t]]
            amax = np.abs(x[i].reshape(4, 128)).max(axis=1)
            for blk in range(4):
                m, _ = np.frexp(s[blk])
                assert m == 0.5, s[blk]  # a power of two
                if amax[blk] == 0:
                    assert s[blk] == 2.0 ** -28 and np.all(vals[blk] == 0)
                else:
                    # the smallest power of two >= amax / 448: amax / s lies in (224, 448], and
                    # its e4m3 code in [224, 448] (just above 224 the code step is 16)
                    assert amax[blk] / 448 <= s[blk] < 2 * amax[blk] / 448
                    assert 224 <= np.abs(vals[blk]).max() <= 448
                    # every code is the e4m3 rounding of x / s (relative error <= 2^-4)
                    xs = x[i].reshape(4, 128)[blk] / s[blk]
                    assert np.all(np.abs(vals[blk] - xs) <= np.abs(xs) * 2.0 ** -4 + 2.0 ** -10)
            assert np.array_equal(rope2[pg[b, t], rw[b, t]], rn[i])
    s1 = scl2[pg[0, 1], rw[0, 1]]
    v1 = decode_e4m3(lat2[pg[0, 1], rw[0, 1]]).reshape(4, 128)
    assert s1[0] == 1.0 and v1[0, 5] == 288.0 and np.count_nonzero(v1[0]) == 1
    assert s1[1] == 2.0 ** -7 and v1[1, 2] == -448.0


def test_write_skips_tokens_without_a_slot():
    # seq 0: L=1 < n_new=3, so positions -2, -1 have no slot and position 0 goes to
    # page 2 row 0; seq 1: L=6, positions 3, 4, 5 are blocks 0, 1, 1 -> page 1 row 3,
    # then block-table entry 9, outside a pool of 4 pages (skipped)
    bt = np.array([[2, 0], [1, 9]])
    pages, rows = write_positions([1, 6], 3, bt, 4, num_pages=4)
    assert pages.tolist() == [[-1, -1, 2], [1, -1, -1]] and rows[0, 2] == 0 and rows[1, 0] == 3
    cache = np.zeros((4, 4, 1, 8), np.uint8)
    x = np.ones((6, 1, 8), np.float32)
    out = write_kv_e4m3(cache, x, [1, 6], 3, bt, np.ones((2, 1), np.float32))
    written = {(int(p), int(r)) for p, r in zip(*np.nonzero(out.any(axis=(2, 3))))}
    assert written == {(2, 0), (1, 3)}
