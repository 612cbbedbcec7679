"""Pins of the fp64 oracle against facts fixed by the pages and by
mathematics (no GPU). Each pin is written so that a plausible slip in the
oracle (a dropped descale, an off-by-one in the causal limit, a transposed
head packing, a wrong sign, a bad table entry) fails at least one of them;
``test_planted_mistakes_are_caught`` plants such slips in copies of the
oracle and checks exactly that."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import brute, formats, merge

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F8 = torch.float8_e4m3fn


# ----------------------------------------------------------------------------
# tiny random inputs in the tensor contract (numpy, no GPU)
# ----------------------------------------------------------------------------
FINITE_CODES = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def tiny_case(rng, *, num_seqs=2, q_len=1, h_q=4, h_k=2, d=8, ps=4, lens=(5, 11), q_fmt="bf16", pages=None,
              code_span=(0x20, 0x50)):
    """Random codes around unit magnitude (so the softmax is not one-hot);
    a shuffled pool with NaN-poisoned unused pages and tail rows."""
    lens = np.asarray(lens, dtype=np.int32)
    blocks = [-(-int(L) // ps) for L in lens]
    max_blocks = max(1, max(blocks))
    used = sum(blocks)
    num_pages = pages or used + 3
    perm = rng.permutation(num_pages)
    bt = np.zeros((num_seqs, max_blocks), np.int32)
    cur = 0
    for b, nb in enumerate(blocks):
        bt[b, :nb] = perm[cur:cur + nb]
        bt[b, nb:] = perm[-1]
        cur += nb

    def cache():
        mag = rng.integers(code_span[0], code_span[1], size=(num_pages, ps, h_k, d), dtype=np.uint8)
        sign = (rng.random((num_pages, ps, h_k, d)) < 0.5).astype(np.uint8) << 7
        c = mag | sign
        c[perm[used:]] = 0x7F
        for b, L in enumerate(lens):  # tail rows of the last page
            if L % ps:
                c[bt[b, blocks[b] - 1], L % ps:] = 0x7F
        return c

    k, v = cache(), cache()
    if q_fmt == "bf16":
        q = bf16_bits(rng.standard_normal((num_seqs * q_len, h_q, d)))
    else:
        q = rng.choice(FINITE_CODES[(FINITE_CODES & 0x7F) < 0x58], size=(num_seqs * q_len, h_q, d))
    qd = (rng.random((num_seqs, h_k)) + 0.5).astype(np.float32)
    kd = (rng.random((num_seqs, h_k)) + 0.5).astype(np.float32)
    vd = (rng.random((num_seqs, h_k)) + 0.5).astype(np.float32)
    return dict(q=q, k_cache=k, v_cache=v, block_table=bt, seq_lens=lens, q_descale=qd, k_descale=kd,
                v_descale=vd, q_len=q_len, h_k=h_k)


def run_oracle(c, fn=None, **kw):
    fn = fn or A.decode_attention
    return fn(c["q"], c["k_cache"], c["v_cache"], c["block_table"], c["seq_lens"], c["q_descale"],
              c["k_descale"], c["v_descale"], q_len=c["q_len"], h_k=c["h_k"], **kw)


def run_brute(c, q_fmt, **kw):
    return brute.brute_decode_attention(
        c["q"].tolist(), q_fmt, c["k_cache"].tolist(), c["v_cache"].tolist(), c["block_table"].tolist(),
        c["seq_lens"].tolist(), c["q_descale"].tolist(), c["k_descale"].tolist(), c["v_descale"].tolist(),
        c["q_len"], c["h_k"], kw["softmax_scale"], kw["o_scale"], kw["causal"])


def torch_decode_e4m3(codes):
    """Decode via torch's own float8_e4m3fn cast (a library routine)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(F8).double().numpy()


# ----------------------------------------------------------------------------
# formats
# ----------------------------------------------------------------------------
def test_e4m3_golden_codes():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e4m3_codes.txt")) if ln.strip() and ln[0] != "#"]
    assert len(rows) >= 14
    for code, val in rows:
        got = formats.E4M3_TABLE[int(code, 16)]
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), (code, got, val)


def test_e4m3_table_properties():
    t = formats.E4M3_TABLE
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "finite positive codes must increase strictly"
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F]), "sign bit flips the value"
    assert np.isnan(t).sum() == 2
    assert np.nanmax(np.abs(t)) == 448.0
    assert len(set(np.abs(t[np.isfinite(t)]).tolist())) == 127  # +-0 coincide


def test_e4m3_table_matches_torch_cast():
    ref = torch_decode_e4m3(np.arange(256, dtype=np.uint8))
    t = formats.E4M3_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(ref[fin], t[fin])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint64).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(formats.decode_bf16(bits), ref)


def test_e2m1_golden_codes():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "e2m1_codes.txt")) if ln.strip() and ln[0] != "#"]
    assert len(rows) == 16
    for code, val in rows:
        got = formats.E2M1_TABLE[int(code, 16)]
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (code, got, val)


def test_fp4_nibble_order_and_packed_decode():
    # byte i holds element 2i in its low nibble and element 2i+1 in its high nibble
    packed = np.array([[0x21, 0xF7, 0x80]], dtype=np.uint8)
    assert formats.unpack_fp4(packed).tolist() == [[1, 2, 7, 15, 0, 8]]
    assert formats.decode_e2m1_packed(packed).tolist() == [[0.5, 1.0, 6.0, -6.0, 0.0, -0.0]]
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 256, size=(5, 8), dtype=np.uint8)
    ref = [brute.fp4_row_to_floats(r) for r in rows.tolist()]
    assert formats.decode_e2m1_packed(rows).tolist() == ref


def fp4_case(rng, **kw):
    """tiny_case with packed e2m1 K/V (random bytes: every code is finite)."""
    c = tiny_case(rng, **kw)
    for name in ("k_cache", "v_cache"):
        shp = c[name].shape
        c[name] = rng.integers(0, 256, size=shp[:-1] + (shp[-1] // 2,), dtype=np.uint8)
    return c


FP4_CASES = [
    dict(num_seqs=2, q_len=1, h_q=4, h_k=2, d=8, ps=4, lens=(5, 11), q_fmt="e4m3", causal=True),
    dict(num_seqs=2, q_len=3, h_q=4, h_k=2, d=8, ps=8, lens=(9, 3), q_fmt="e4m3", causal=False),
    dict(num_seqs=3, q_len=2, h_q=6, h_k=3, d=16, ps=4, lens=(0, 1, 13), q_fmt="e4m3", causal=True),
]


@pytest.mark.parametrize("case", range(len(FP4_CASES)))
def test_fp4_oracle_matches_brute_force(case):
    cfg = dict(FP4_CASES[case])
    causal = cfg.pop("causal")
    c = fp4_case(np.random.default_rng(900 + case), **cfg)
    kw = dict(softmax_scale=0.37, o_scale=1.25, causal=causal)
    o, lse = run_oracle(c, kv_format="e2m1", **kw)
    ob, lb = brute.brute_decode_attention(
        c["q"].tolist(), "e4m3", c["k_cache"].tolist(), c["v_cache"].tolist(), c["block_table"].tolist(),
        c["seq_lens"].tolist(), c["q_descale"].tolist(), c["k_descale"].tolist(), c["v_descale"].tolist(),
        c["q_len"], c["h_k"], kw["softmax_scale"], kw["o_scale"], kw["causal"], kv_fmt="e2m1")
    assert o.shape[-1] == cfg["d"] and np.all(np.isfinite(o))
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_array_equal(fin, np.isfinite(np.array(lb)))
    np.testing.assert_allclose(lse[fin], np.array(lb)[fin], rtol=0, atol=1e-12)


def test_fp4_equals_e4m3_on_the_same_values():
    # every e2m1 value is an e4m3 value: re-encoding the unpacked codes as the
    # e4m3 bytes of the same values (found by lookup in the e4m3 table) must
    # give the identical result through the e4m3 path
    c = fp4_case(np.random.default_rng(77), num_seqs=2, q_len=2, h_q=4, h_k=2, d=16, ps=4, lens=(6, 13),
                 q_fmt="e4m3")
    mag = {float(formats.E4M3_TABLE[m]): m for m in range(0x7F)}  # finite non-negative e4m3 codes
    lut = np.array([mag[abs(float(formats.E2M1_TABLE[c]))] | (0x80 if c & 8 else 0) for c in range(16)],
                   dtype=np.uint8)
    c8 = dict(c)
    c8["k_cache"] = lut[formats.unpack_fp4(c["k_cache"])]
    c8["v_cache"] = lut[formats.unpack_fp4(c["v_cache"])]
    assert np.array_equal(formats.decode_e4m3(c8["k_cache"]), formats.decode_e2m1_packed(c["k_cache"]))
    kw = dict(softmax_scale=0.29, causal=True)
    o4, l4 = run_oracle(c, kv_format="e2m1", **kw)
    o8, l8 = run_oracle(c8, **kw)
    assert np.array_equal(o4, o8) and np.array_equal(l4, l8)


# ----------------------------------------------------------------------------
# attention: brute force, special cases, textbook routine
# ----------------------------------------------------------------------------
CASES = [
    dict(num_seqs=2, q_len=1, h_q=4, h_k=2, d=8, ps=4, lens=(5, 11), q_fmt="bf16", causal=True),
    dict(num_seqs=2, q_len=3, h_q=4, h_k=1, d=8, ps=4, lens=(7, 10), q_fmt="bf16", causal=True),
    dict(num_seqs=2, q_len=3, h_q=4, h_k=2, d=8, ps=8, lens=(9, 3), q_fmt="e4m3", causal=False),
    dict(num_seqs=3, q_len=2, h_q=6, h_k=3, d=16, ps=4, lens=(0, 1, 13), q_fmt="e4m3", causal=True),
    dict(num_seqs=1, q_len=4, h_q=2, h_k=1, d=8, ps=4, lens=(2,), q_fmt="bf16", causal=True),  # L < q_len
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_oracle_matches_brute_force(case):
    cfg = dict(CASES[case])
    causal = cfg.pop("causal")
    rng = np.random.default_rng(100 + case)
    c = tiny_case(rng, **cfg)
    kw = dict(softmax_scale=0.37, o_scale=1.25, causal=causal)
    o, lse = run_oracle(c, **kw)
    ob, lb = run_brute(c, cfg["q_fmt"], **kw)
    assert np.all(np.isfinite(o))
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(np.array(lb)))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], np.array(lb)[fin], rtol=0, atol=1e-12)


def test_empty_rows_are_zero_and_minus_inf():
    rng = np.random.default_rng(7)
    c = tiny_case(rng, num_seqs=2, q_len=3, h_q=2, h_k=1, lens=(0, 2))
    o, lse = run_oracle(c, softmax_scale=0.5, causal=True)
    assert np.all(o[:3] == 0) and np.all(np.isneginf(lse[0]))
    # seq 1, L = 2, q_len = 3: row qi sees keys 0 .. qi-1 -> qi = 0 sees none
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[1, 0, :2]))
    assert np.all(np.isfinite(lse[1, 0, 2:]))


def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(8)
    c = tiny_case(rng, num_seqs=1, h_q=4, h_k=2, lens=(1,))
    o, lse = run_oracle(c, softmax_scale=0.3, o_scale=2.0)
    page = c["block_table"][0, 0]
    for g in range(2):
        v0 = torch_decode_e4m3(c["v_cache"][page, 0, g]) * np.float64(c["v_descale"][0, g])
        k0 = torch_decode_e4m3(c["k_cache"][page, 0, g]) * np.float64(c["k_descale"][0, g])
        for hr in range(2):
            np.testing.assert_array_equal(o[0, g * 2 + hr], 2.0 * v0)
            q = torch.from_numpy(c["q"][0, g * 2 + hr].view(np.int16)).view(torch.bfloat16).double().numpy()
            assert abs(lse[0, g, hr] - 0.3 * float(q @ k0)) < 1e-12


def test_constant_v_returns_that_value():
    rng = np.random.default_rng(9)
    c = tiny_case(rng, num_seqs=2, q_len=2, h_q=4, h_k=2, lens=(6, 9))
    c["v_cache"][:] = 0x3C  # 1.5 everywhere, poison included (never read)
    o, _ = run_oracle(c, softmax_scale=0.7, o_scale=1.0, causal=True)
    vd = np.repeat(np.repeat(c["v_descale"].astype(np.float64), 2, axis=1)[:, None, :], 2, axis=1)
    np.testing.assert_allclose(o, 1.5 * vd.reshape(4, 4)[:, :, None] * np.ones(8), rtol=1e-14, atol=0)


def test_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(10)
    c = tiny_case(rng, num_seqs=1, q_len=3, h_q=2, h_k=1, lens=(10,))
    c["q"][:] = 0
    o, lse = run_oracle(c, softmax_scale=1.0, causal=True)
    V = torch_decode_e4m3(c["v_cache"][c["block_table"][0]][:, :, 0].reshape(-1, 8)[:10]) * np.float64(c["v_descale"][0, 0])
    for qi in range(3):
        vis = 10 - 3 + qi + 1
        for hr in range(2):
            np.testing.assert_allclose(o[qi, hr], V[:vis].mean(axis=0), rtol=1e-13, atol=1e-15)
            assert abs(lse[0, 0, qi * 2 + hr] - math.log(vis)) < 1e-13


def test_two_keys_sigmoid_weight():
    rng = np.random.default_rng(11)
    c = tiny_case(rng, num_seqs=1, h_q=1, h_k=1, lens=(2,))
    o, lse = run_oracle(c, softmax_scale=0.9)
    page = c["block_table"][0, 0]
    q = torch.from_numpy(c["q"][0, 0].view(np.int16)).view(torch.bfloat16).double().numpy()
    K = torch_decode_e4m3(c["k_cache"][page, :2, 0]) * np.float64(c["k_descale"][0, 0])
    V = torch_decode_e4m3(c["v_cache"][page, :2, 0]) * np.float64(c["v_descale"][0, 0])
    s0, s1 = 0.9 * (K @ q)
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    np.testing.assert_allclose(o[0, 0], w0 * V[0] + (1 - w0) * V[1], rtol=1e-13, atol=1e-15)
    assert abs(lse[0, 0, 0] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-13


@pytest.mark.parametrize("q_len,causal,q_fmt", [(1, True, "bf16"), (4, True, "bf16"), (4, False, "e4m3"),
                                                (3, True, "e4m3")])
def test_oracle_matches_torch_sdpa_fp64(q_len, causal, q_fmt):
    rng = np.random.default_rng(12 + q_len)
    h_q, h_k, d, ps = 8, 2, 16, 8
    c = tiny_case(rng, num_seqs=3, q_len=q_len, h_q=h_q, h_k=h_k, d=d, ps=ps, lens=(23, 40, 9), q_fmt=q_fmt)
    scale = 0.21
    o, lse = run_oracle(c, softmax_scale=scale, o_scale=0.75, causal=causal)
    h_r = h_q // h_k
    for b, L in enumerate(c["seq_lens"]):
        pages = c["block_table"][b, : -(-L // ps)]
        K = torch.from_numpy(torch_decode_e4m3(c["k_cache"][pages].reshape(-1, h_k, d)[:L]))
        V = torch.from_numpy(torch_decode_e4m3(c["v_cache"][pages].reshape(-1, h_k, d)[:L]))
        K = K * torch.from_numpy(c["k_descale"][b].astype(np.float64))[None, :, None]
        V = V * torch.from_numpy(c["v_descale"][b].astype(np.float64))[None, :, None]
        qb = c["q"][b * q_len:(b + 1) * q_len]
        if q_fmt == "bf16":
            Q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).double()
        else:
            Q = torch.from_numpy(torch_decode_e4m3(qb)) * torch.from_numpy(
                np.repeat(c["q_descale"][b].astype(np.float64), h_r))[None, :, None]
        # (q_len, h_q, d) -> heads first; K/V heads repeated for GQA
        Qh = Q.permute(1, 0, 2)
        Kh = K.permute(1, 0, 2).repeat_interleave(h_r, dim=0)
        Vh = V.permute(1, 0, 2).repeat_interleave(h_r, dim=0)
        qi = torch.arange(q_len)[:, None]
        j = torch.arange(L)[None, :]
        allowed = (j <= L - q_len + qi) if (causal and q_len > 1) else torch.ones(q_len, L, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(Qh, Kh, Vh, attn_mask=allowed, scale=scale)
        ref_lse = torch.logsumexp((scale * Qh @ Kh.transpose(1, 2)).masked_fill(~allowed, -math.inf), dim=-1)
        np.testing.assert_allclose(o[b * q_len:(b + 1) * q_len], 0.75 * ref.permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-13)
        # lse (h_k, q_len*h_r) qi-major  <->  ref_lse (h_q, q_len)
        packed = ref_lse.view(h_k, h_r, q_len).permute(0, 2, 1).reshape(h_k, q_len * h_r)
        np.testing.assert_allclose(lse[b], packed.numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------
def _dense_rows(c, b, g, scale=1.0):
    """(qrows, K, V, limits) of one (seq, head) via the oracle's own gather."""
    q_len, h_k = c["q_len"], c["h_k"]
    h_q = c["q"].shape[1]
    h_r = h_q // h_k
    L = int(c["seq_lens"][b])
    K = formats.decode_e4m3(A.gather_tokens(c["k_cache"], c["block_table"][b], L, g)) * float(c["k_descale"][b, g])
    V = formats.decode_e4m3(A.gather_tokens(c["v_cache"], c["block_table"][b], L, g)) * float(c["v_descale"][b, g])
    rows = formats.decode_bf16(c["q"][b * q_len:(b + 1) * q_len, g * h_r:(g + 1) * h_r]).reshape(q_len * h_r, -1)
    return rows, K, V, A.row_limits(L, q_len, h_r, True)


@pytest.mark.parametrize("seed", range(6))
def test_split_invariance(seed):
    rng = np.random.default_rng(200 + seed)
    c = tiny_case(rng, num_seqs=2, q_len=3, h_q=4, h_k=2, d=16, ps=4, lens=(37, 29))
    for b in range(2):
        for g in range(2):
            rows, K, V, lim = _dense_rows(c, b, g)
            L = K.shape[0]
            cuts = sorted(set(rng.integers(1, L, size=rng.integers(1, 6)).tolist()))
            bounds = list(zip([0] + cuts, cuts + [L]))
            o1, l1 = A.attend(rows, K, V, lim, 0.45, 1.5)
            o2, l2 = merge.split_attend(rows, K, V, lim, 0.45, 1.5, bounds)
            np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
            np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_merge_degenerate_cases():
    o, lse = merge.merge_partials([np.ones(3)], [0.5], [2.0], o_scale=1.0)
    np.testing.assert_allclose(o, np.ones(3) / 2.0)
    assert lse == 0.5 + math.log(2.0)
    o, lse = merge.merge_partials([np.zeros(3), np.zeros(3)], [-np.inf, -np.inf], [0.0, 0.0])
    assert np.all(o == 0) and lse == -np.inf
    # a chunk wholly past a row's causal limit contributes nothing
    o, lse = merge.merge_partials([np.full(2, 3.0), np.zeros(2)], [1.0, -np.inf], [1.5, 0.0])
    np.testing.assert_allclose(o, np.full(2, 2.0))
    assert abs(lse - (1.0 + math.log(1.5))) < 1e-15


def test_page_permutation_invariance():
    rng = np.random.default_rng(300)
    c = tiny_case(rng, num_seqs=3, q_len=2, h_q=4, h_k=2, d=8, ps=4, lens=(13, 4, 21))
    o1, l1 = run_oracle(c, softmax_scale=0.4)
    P = c["k_cache"].shape[0]
    perm = rng.permutation(P)  # physical page p moves to slot perm[p]
    c2 = dict(c)
    for name in ("k_cache", "v_cache"):
        moved = np.empty_like(c[name])
        moved[perm] = c[name]
        c2[name] = moved
    c2["block_table"] = perm[c["block_table"]].astype(np.int32)
    o2, l2 = run_oracle(c2, softmax_scale=0.4)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_causal_rows_equal_shorter_single_token_decodes():
    rng = np.random.default_rng(400)
    q_len, h_q, h_k = 4, 4, 2
    c = tiny_case(rng, num_seqs=2, q_len=q_len, h_q=h_q, h_k=h_k, d=8, ps=4, lens=(15, 9))
    o, lse = run_oracle(c, softmax_scale=0.5, causal=True)
    h_r = h_q // h_k
    for b, L in enumerate(c["seq_lens"]):
        for qi in range(q_len):
            c1 = dict(c, q=c["q"][b * q_len + qi:b * q_len + qi + 1], q_len=1, block_table=c["block_table"][b:b + 1],
                      seq_lens=np.array([L - q_len + qi + 1], np.int32), q_descale=c["q_descale"][b:b + 1],
                      k_descale=c["k_descale"][b:b + 1], v_descale=c["v_descale"][b:b + 1])
            o1, l1 = run_oracle(c1, softmax_scale=0.5)
            np.testing.assert_array_equal(o[b * q_len + qi], o1[0])
            np.testing.assert_array_equal(lse[b, :, qi * h_r:(qi + 1) * h_r], l1[0])


def test_block_mode_rows_equal_full_single_token_decodes():
    rng = np.random.default_rng(401)
    q_len, h_q, h_k = 3, 4, 2
    c = tiny_case(rng, num_seqs=2, q_len=q_len, h_q=h_q, h_k=h_k, d=8, ps=4, lens=(12, 7))
    o, lse = run_oracle(c, softmax_scale=0.5, causal=False)
    for b, L in enumerate(c["seq_lens"]):
        for qi in range(q_len):
            c1 = dict(c, q=c["q"][b * q_len + qi:b * q_len + qi + 1], q_len=1, block_table=c["block_table"][b:b + 1],
                      seq_lens=np.array([L], np.int32), q_descale=c["q_descale"][b:b + 1],
                      k_descale=c["k_descale"][b:b + 1], v_descale=c["v_descale"][b:b + 1])
            o1, _ = run_oracle(c1, softmax_scale=0.5)
            np.testing.assert_array_equal(o[b * q_len + qi], o1[0])


def test_gqa_equals_mha_with_replicated_kv():
    rng = np.random.default_rng(500)
    q_len, h_q, h_k = 2, 6, 2
    h_r = h_q // h_k
    c = tiny_case(rng, num_seqs=2, q_len=q_len, h_q=h_q, h_k=h_k, d=8, ps=4, lens=(10, 6), q_fmt="e4m3")
    o, lse = run_oracle(c, softmax_scale=0.3, causal=True)
    cm = dict(c, h_k=h_q, k_cache=np.repeat(c["k_cache"], h_r, axis=2), v_cache=np.repeat(c["v_cache"], h_r, axis=2),
              q_descale=np.repeat(c["q_descale"], h_r, axis=1), k_descale=np.repeat(c["k_descale"], h_r, axis=1),
              v_descale=np.repeat(c["v_descale"], h_r, axis=1))
    om, lm = run_oracle(cm, softmax_scale=0.3, causal=True)
    np.testing.assert_array_equal(o, om)
    # MHA lse (b, h_q, q_len) vs GQA packed (b, h_k, q_len*h_r)
    np.testing.assert_array_equal(lse, lm.reshape(2, h_k, h_r, q_len).transpose(0, 1, 3, 2).reshape(2, h_k, -1))


def test_descales_broadcast_and_fold():
    rng = np.random.default_rng(501)
    c = tiny_case(rng, num_seqs=2, q_len=1, h_q=4, h_k=2, d=8, ps=4, lens=(9, 5), q_fmt="e4m3")
    for name in ("q_descale", "k_descale", "v_descale"):
        per_tensor = dict(c, **{name: np.float32(0.625)})
        full = dict(c, **{name: np.full((2, 2), 0.625, np.float32)})
        np.testing.assert_array_equal(run_oracle(per_tensor, softmax_scale=0.3)[0],
                                      run_oracle(full, softmax_scale=0.3)[0])
    # scaling K's descale by t is the same as scaling the softmax scale by t
    ck = dict(c, k_descale=c["k_descale"] * np.float32(2.0))
    o1, l1 = run_oracle(ck, softmax_scale=0.3)
    o2, l2 = run_oracle(c, softmax_scale=0.6)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------------
# latent-record variant
# ----------------------------------------------------------------------------
def test_mla_matches_sdpa_on_assembled_keys():
    rng = np.random.default_rng(600)
    P, ps, h_q, q_len = 6, 4, 4, 2
    lens = np.array([7, 13], np.int32)
    bt = np.array([[3, 0, 5, 5], [1, 4, 2, 5]], np.int32)
    latent = rng.choice(FINITE_CODES[(FINITE_CODES & 0x7F) < 0x48], size=(P, ps, 1, 512)).astype(np.uint8)
    rope = bf16_bits(rng.standard_normal((P, ps, 1, 64)))
    scales = (rng.random((P, ps, 1, 4)) * 0.05 + 0.01).astype(np.float32)
    q = bf16_bits(rng.standard_normal((2 * q_len, h_q, 576)) * 0.1)
    scale = 1.0 / 24.0
    o, lse = A.mla_decode_attention(q, latent, rope, scales, bt, lens, q_len=q_len, softmax_scale=scale,
                                    o_scale=1.0, causal=True)
    for b, L in enumerate(lens):
        toks = [(bt[b, j // ps], j % ps) for j in range(L)]
        lat = np.stack([torch_decode_e4m3(latent[p, r, 0]) * np.repeat(scales[p, r, 0].astype(np.float64), 128)
                        for p, r in toks])
        rp = np.stack([torch.from_numpy(rope[p, r, 0].view(np.int16)).view(torch.bfloat16).double().numpy()
                       for p, r in toks])
        K = torch.from_numpy(np.concatenate([lat, rp], axis=1))[None]
        V = torch.from_numpy(lat)[None]
        Q = torch.from_numpy(q[b * q_len:(b + 1) * q_len].view(np.int16)).view(torch.bfloat16).double()
        Q = Q.reshape(1, q_len * h_q, 576)  # rows n = qi*h_q + h
        qi = torch.arange(q_len * h_q)[:, None] // h_q
        allowed = torch.arange(L)[None, :] <= L - q_len + qi
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=allowed, scale=scale)
        np.testing.assert_allclose(o[b * q_len:(b + 1) * q_len].reshape(-1, 512), ref[0].numpy(), rtol=1e-12,
                                   atol=1e-14)
        ref_lse = torch.logsumexp((scale * Q @ K.transpose(1, 2)).masked_fill(~allowed, -math.inf), -1)
        np.testing.assert_allclose(lse[b, 0], ref_lse[0].numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# the pins catch planted mistakes (mistakes planted in copies of the oracle)
# ----------------------------------------------------------------------------
def _pins_pass(oracle_fn):
    """Re-run the brute-force and SDPA-style pins against ``oracle_fn``;
    True if every one still passes."""
    try:
        for case in range(len(CASES)):
            cfg = dict(CASES[case])
            causal = cfg.pop("causal")
            c = tiny_case(np.random.default_rng(100 + case), **cfg)
            kw = dict(softmax_scale=0.37, o_scale=1.25, causal=causal)
            o, lse = run_oracle(c, fn=oracle_fn, **kw)
            ob, lb = run_brute(c, cfg["q_fmt"], **kw)
            np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
            lb = np.array(lb)
            np.testing.assert_array_equal(np.isinf(lse), np.isinf(lb))
            np.testing.assert_allclose(lse[np.isfinite(lse)], lb[np.isfinite(lb)], rtol=0, atol=1e-12)
        return True
    except AssertionError:
        return False


def test_planted_mistakes_are_caught(monkeypatch):
    assert _pins_pass(A.decode_attention)
    import importlib

    mutants = {
        "no k descale": lambda s: s.replace("* kd[b, g]", ""),
        "no v descale": lambda s: s.replace("* vd[b, g]", ""),
        "no o_scale": lambda s: s.replace("out[n] = o_scale * ", "out[n] = "),
        "causal off by one": lambda s: s.replace("return L - q_len + qi", "return L - q_len + qi + 1"),
        "head-major packing": lambda s: s.replace("qi = np.arange(q_len * h_r) // h_r",
                                                  "qi = np.arange(q_len * h_r) % q_len"),
        "lse without max": lambda s: s.replace("lse[n] = m + np.log(den)", "lse[n] = np.log(den)"),
        "wrong exp sign": lambda s: s.replace("w = np.exp(s - m)", "w = np.exp(m - s)"),
        "transposed score": lambda s: s.replace("(K[:vis] @ qrows[n])", "(K[:vis] @ qrows[(n + 1) % n_rows])"),
        "no q descale": lambda s: s.replace("* qd[b, g]\n", "\n"),
    }
    src = open(A.__file__).read()
    for name, mut in mutants.items():
        msrc = mut(src)
        assert msrc != src, f"mutant {name!r} did not change the source"
        mod = type(A)("oracle_mutant")
        mod.__dict__["__name__"] = "oracle.mutant"
        mod.__dict__["__package__"] = "oracle"
        exec(compile(msrc, "mutant", "exec"), mod.__dict__)
        assert not _pins_pass(mod.decode_attention), f"planted mistake {name!r} survived every pin"


def test_fp6_golden_codes():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "fp6_codes.txt")) if ln.strip() and ln[0] != "#"]
    assert len(rows) == 33
    tables = {"e2m3": formats.E2M3_TABLE, "e3m2": formats.E3M2_TABLE}
    for fmt, code, val in rows:
        got = tables[fmt][int(code, 16)]
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)), (fmt, code, got, val)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_value_set_properties(fmt):
    t = {"e2m3": formats.E2M3_TABLE, "e3m2": formats.E3M2_TABLE}[fmt]
    pos = t[:32]
    assert np.all(np.isfinite(t)) and np.all(np.diff(pos) > 0)  # no inf/NaN, strictly increasing
    assert np.array_equal(t[32:], -pos)  # sign-magnitude
    assert pos[-1] == {"e2m3": 7.5, "e3m2": 28.0}[fmt] and pos[1] == {"e2m3": 0.125, "e3m2": 0.0625}[fmt]
    # every fp6 value is an e4m3 value (torch's float8_e4m3fn cast returns it unchanged)
    back = torch.from_numpy(t.copy()).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(back, t)


def test_fp6_packing_golden_and_decode():
    for ln in open(os.path.join(GOLDEN, "fp6_pack.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        b, c = ln.split("|")
        packed = np.array([[int(x, 16) for x in b.split()]], dtype=np.uint8)
        assert formats.unpack_fp6(packed).tolist() == [[int(x, 16) for x in c.split()]]
    rng = np.random.default_rng(4)
    rows = rng.integers(0, 256, size=(6, 12), dtype=np.uint8)
    for fmt, dec in (("e2m3", formats.decode_e2m3_packed), ("e3m2", formats.decode_e3m2_packed)):
        ref = [brute.fp6_row_to_floats(r, fmt) for r in rows.tolist()]
        assert dec(rows).tolist() == ref


def fp6_case(rng, **kw):
    """tiny_case with packed fp6 K/V (random bytes: every code is finite)."""
    c = tiny_case(rng, **kw)
    for name in ("k_cache", "v_cache"):
        shp = c[name].shape
        c[name] = rng.integers(0, 256, size=shp[:-1] + (shp[-1] * 3 // 4,), dtype=np.uint8)
    return c


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("case", range(len(FP4_CASES)))
def test_fp6_oracle_matches_brute_force(case, fmt):
    cfg = dict(FP4_CASES[case])
    causal = cfg.pop("causal")
    c = fp6_case(np.random.default_rng(950 + case), **cfg)
    kw = dict(softmax_scale=0.21, o_scale=0.8, causal=causal)
    o, lse = run_oracle(c, kv_format=fmt, **kw)
    ob, lb = brute.brute_decode_attention(
        c["q"].tolist(), "e4m3", c["k_cache"].tolist(), c["v_cache"].tolist(), c["block_table"].tolist(),
        c["seq_lens"].tolist(), c["q_descale"].tolist(), c["k_descale"].tolist(), c["v_descale"].tolist(),
        c["q_len"], c["h_k"], kw["softmax_scale"], kw["o_scale"], kw["causal"], kv_fmt=fmt)
    assert o.shape[-1] == cfg["d"] and np.all(np.isfinite(o))
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_array_equal(fin, np.isfinite(np.array(lb)))
    np.testing.assert_allclose(lse[fin], np.array(lb)[fin], rtol=0, atol=1e-12)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_fp6_equals_e4m3_on_the_same_values(fmt):
    c = fp6_case(np.random.default_rng(78), num_seqs=2, q_len=2, h_q=4, h_k=2, d=16, ps=4, lens=(6, 13),
                 q_fmt="e4m3")
    table = {"e2m3": formats.E2M3_TABLE, "e3m2": formats.E3M2_TABLE}[fmt]
    mag = {float(formats.E4M3_TABLE[m]): m for m in range(0x7F)}
    lut = np.array([mag[abs(float(table[c]))] | (0x80 if c & 0x20 else 0) for c in range(64)], dtype=np.uint8)
    c8 = dict(c)
    c8["k_cache"] = lut[formats.unpack_fp6(c["k_cache"])]
    c8["v_cache"] = lut[formats.unpack_fp6(c["v_cache"])]
    kw = dict(softmax_scale=0.29, causal=True)
    o6, l6 = run_oracle(c, kv_format=fmt, **kw)
    o8, l8 = run_oracle(c8, **kw)
    assert np.array_equal(o6, o8) and np.array_equal(l6, l8)



def test_nvfp4_kernel_values_closed_forms():
    from oracle.producers import nvfp4_kernel_values
    # one row of 16 codes per case, one scale byte each
    def val(code, scale_byte):
        packed = np.array([[code | (code << 4)] * 8], dtype=np.uint8)
        return nvfp4_kernel_values(packed, np.array([[scale_byte]], dtype=np.uint8))[0, 0]
    # the page's bound: code 6.0 times scale 448 times 2^-3 = 336, not an e4m3
    # value; halfway between 320 (even code 0x7A) and 352 (0x7B): ties to even
    assert val(0x7, 0x7E) == 320.0
    assert val(0xF, 0x7E) == -320.0
    assert val(0x2, 0x38) == 0.125                   # 1.0 * 1.0 / 8, exact
    assert val(0x1, 0x08) == 0.0                     # 0.5 * 2^-6 / 8 = 2^-10: half the smallest subnormal, ties to 0
    assert val(0x3, 0x08) == 2.0 ** -8               # 1.5 * 2^-9: halfway between subnormal codes 1 and 2, ties to 2
    assert val(0x5, 0x3C) == 0.5625                  # 3 * 1.5 / 8 = 0.5625 = 1.125 * 2^-1, exact


def test_nvfp4_rounding_matches_torch_cast():
    from oracle.producers import nvfp4_kernel_values
    rng = np.random.default_rng(21)
    packed = rng.integers(0, 256, size=(64, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, size=(64, 8), dtype=np.uint8)  # finite, non-negative scales
    got = nvfp4_kernel_values(packed, scales)
    prod = formats.E2M1_TABLE[formats.unpack_fp4(packed)] * np.repeat(formats.E4M3_TABLE[scales], 16, axis=-1) / 8
    ref = torch.from_numpy(prod.astype(np.float32)).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(got, ref)


def nvfp4_case(rng, **kw):
    c = fp4_case(rng, **kw)
    for name in ("k_scale", "v_scale"):
        shp = c["k_cache"].shape
        c[name] = rng.integers(0x20, 0x60, size=shp[:-1] + (shp[-1] * 2 // 16,), dtype=np.uint8)
    return c


NVFP4_CASES = [
    dict(num_seqs=2, q_len=1, h_q=4, h_k=2, d=16, ps=4, lens=(5, 11), q_fmt="e4m3", causal=True),
    dict(num_seqs=2, q_len=3, h_q=4, h_k=2, d=32, ps=8, lens=(9, 3), q_fmt="e4m3", causal=False),
]


@pytest.mark.parametrize("case", range(len(NVFP4_CASES)))
def test_nvfp4_oracle_matches_brute_force(case):
    cfg = dict(NVFP4_CASES[case])
    causal = cfg.pop("causal")
    c = nvfp4_case(np.random.default_rng(990 + case), **cfg)
    kw = dict(softmax_scale=0.33, o_scale=1.1, causal=causal)
    o, lse = run_oracle(c, kv_format="nvfp4", k_scale=c["k_scale"], v_scale=c["v_scale"], **kw)
    ob, lb = brute.brute_decode_attention(
        c["q"].tolist(), "e4m3", c["k_cache"].tolist(), c["v_cache"].tolist(), c["block_table"].tolist(),
        c["seq_lens"].tolist(), c["q_descale"].tolist(), c["k_descale"].tolist(), c["v_descale"].tolist(),
        c["q_len"], c["h_k"], kw["softmax_scale"], kw["o_scale"], kw["causal"], kv_fmt="nvfp4",
        k_scale=c["k_scale"].tolist(), v_scale=c["v_scale"].tolist())
    assert o.shape[-1] == cfg["d"] and np.all(np.isfinite(o))
    np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], np.array(lb)[fin], rtol=0, atol=1e-12)


def test_nvfp4_with_unit_group_scales_is_the_fp4_path():
    # scale 8.0 (e4m3 0x50) times 2^-3 is 1: every kernel value is the e2m1 value itself
    c = nvfp4_case(np.random.default_rng(79), num_seqs=2, q_len=2, h_q=4, h_k=2, d=32, ps=4, lens=(6, 13),
                   q_fmt="e4m3")
    c["k_scale"][:] = 0x50
    c["v_scale"][:] = 0x50
    kw = dict(softmax_scale=0.29, causal=True)
    on, ln = run_oracle(c, kv_format="nvfp4", k_scale=c["k_scale"], v_scale=c["v_scale"], **kw)
    o4, l4 = run_oracle(c, kv_format="e2m1", **kw)
    assert np.array_equal(on, o4) and np.array_equal(ln, l4)
