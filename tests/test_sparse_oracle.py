"""Pins of the sparse slot-list decode oracle (``oracle.sparse``) against
things other than itself: the contiguous latent decode (pinned in
test_oracle.py), the closed form of the attention sink, a pure-Python brute
force, order and split invariance, and the empty cases. CPU only."""

import numpy as np

from oracle import attention as A
from oracle import brute, merge
from oracle.sparse import gather_slots, sparse_decode_attention


def _finite_e4m3(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, c ^ 0x01, c).astype(np.uint8)  # no NaN codes


def _bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def pool(rng, pages, ps):
    return dict(latent=_finite_e4m3(rng, (pages, ps, 1, 512)),
                rope=_bf16_bits(rng, (pages, ps, 1, 64)),
                scales=rng.uniform(0.002, 0.02, size=(pages, ps, 1, 4)).astype(np.float32))


def test_lists_of_a_sequences_own_slots_reproduce_the_contiguous_decode():
    rng = np.random.default_rng(5)
    ps, pages = 16, 12
    p = pool(rng, pages, ps)
    lens = np.array([37, 100, 5])
    bt = np.stack([rng.permutation(pages)[:7] for _ in lens]).astype(np.int32)
    q = _bf16_bits(rng, (3, 16, 576), 0.3)
    o_ref, l_ref = A.mla_decode_attention(q, p["latent"], p["rope"], p["scales"], bt, lens, q_len=1,
                                          softmax_scale=0.05, o_scale=1.1, causal=True)
    width = 128
    slots = np.full((3, width), -1, dtype=np.int32)
    for t, L in enumerate(lens):
        j = np.arange(L)
        slots[t, :L] = bt[t, j // ps] * ps + j % ps
    # the same keys split over the two lists, with padding in between
    s0, s1 = slots.copy(), np.full((3, 64), -1, dtype=np.int32)
    s0[:, 20:40], s1[:, 3:23] = -1, slots[:, 20:40]
    for srcs in ([dict(p, slots=slots)], [dict(p, slots=s0), dict(p, slots=s1)]):
        o, lse = sparse_decode_attention(q, srcs, softmax_scale=0.05, o_scale=1.1)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l_ref[:, 0, :], rtol=0, atol=1e-12)


def test_sink_closed_form():
    rng = np.random.default_rng(6)
    p = pool(rng, 6, 16)
    slots = rng.integers(-1, 6 * 16, size=(2, 40)).astype(np.int32)
    q = _bf16_bits(rng, (2, 16, 576), 0.3)
    sink = rng.uniform(-3, 8, size=16)
    o0, l0 = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.07)
    o1, l1 = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.07, sink=sink)
    np.testing.assert_allclose(l1, np.logaddexp(l0, sink[None, :]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(o1, o0 * np.exp(l0 - l1)[..., None], rtol=0, atol=1e-12)


def test_brute_force_on_tiny_lists():
    rng = np.random.default_rng(7)
    pa, pb = pool(rng, 3, 4), pool(rng, 2, 8)
    sa = np.array([[0, 5, -1, 11, 5], [-1, -1, -1, -1, -1]], dtype=np.int32)  # a duplicate; an empty list
    sb = np.array([[15, -1, 2], [3, 9, -1]], dtype=np.int32)
    q = _bf16_bits(rng, (2, 2, 576), 0.4)
    sink = np.array([0.7, -1.5])
    for sk in (None, sink):
        srcs = [dict(pa, slots=sa), dict(pb, slots=sb)]
        o, lse = sparse_decode_attention(q, srcs, softmax_scale=0.09, o_scale=0.9, sink=sk)
        lists = [{k: v.tolist() for k, v in s.items()} for s in srcs]
        ob, lb = brute.brute_sparse_decode(q.tolist(), lists, 0.09, 0.9, None if sk is None else sk.tolist())
        np.testing.assert_allclose(o, np.array(ob), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(lb), rtol=0, atol=1e-12)


def test_list_order_does_not_matter():
    rng = np.random.default_rng(8)
    p = pool(rng, 5, 16)
    slots = rng.integers(-1, 80, size=(2, 50)).astype(np.int32)
    q = _bf16_bits(rng, (2, 16, 576), 0.3)
    o, lse = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.06)
    perm = slots[:, rng.permutation(50)]
    o2, l2 = sparse_decode_attention(q, [dict(p, slots=perm)], softmax_scale=0.06)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)


def test_tile_partials_merge_with_one_sink_term():
    # the kernel's split: tiles of a list merged with the LSE rule, the sink
    # added once as a partial with O = 0 and l = 1 at max = sink
    rng = np.random.default_rng(9)
    p = pool(rng, 5, 16)
    slots = rng.integers(-1, 80, size=(1, 70)).astype(np.int32)
    q = _bf16_bits(rng, (1, 16, 576), 0.3)
    sink = rng.uniform(-2, 5, size=16)
    o_ref, l_ref = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.06, o_scale=1.3, sink=sink)
    K, V = A.mla_keys_values(gather_slots(p["latent"], slots[0]), gather_slots(p["rope"], slots[0]),
                             gather_slots(p["scales"], slots[0]))
    qf = A._decode_q(q)[0]
    for h in range(16):
        parts = [merge.chunk_partial(qf[h], K, V, b, min(b + 16, len(K)), len(K) - 1, 0.06)
                 for b in range(0, len(K), 16)]
        os_, ms, ls = [x[0] for x in parts], [x[1] for x in parts], [x[2] for x in parts]
        os_.append(np.zeros(512)); ms.append(float(sink[h])); ls.append(1.0)
        o_m, l_m = merge.merge_partials(os_, ms, ls, o_scale=1.3)
        np.testing.assert_allclose(o_m, o_ref[0, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_m, l_ref[0, h], rtol=0, atol=1e-12)


def test_empty_lists():
    rng = np.random.default_rng(10)
    p = pool(rng, 2, 16)
    slots = np.full((2, 8), -1, dtype=np.int32)
    q = _bf16_bits(rng, (2, 16, 576))
    o, lse = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.1)
    assert np.all(o == 0) and np.all(lse == -np.inf)
    sink = rng.uniform(-1, 1, size=16)
    o, lse = sparse_decode_attention(q, [dict(p, slots=slots)], softmax_scale=0.1, sink=sink)
    assert np.all(o == 0) and np.array_equal(lse, np.broadcast_to(sink, (2, 16)))


def test_a_slot_past_the_pool_names_no_key():
    rng = np.random.default_rng(11)
    p = pool(rng, 2, 16)
    q = _bf16_bits(rng, (1, 16, 576))
    past = np.array([[3, 32, 7, 5000]], np.int32)
    neg = np.array([[3, -1, 7, -1]], np.int32)
    o1, l1 = sparse_decode_attention(q, [dict(p, slots=past)], softmax_scale=0.1)
    o2, l2 = sparse_decode_attention(q, [dict(p, slots=neg)], softmax_scale=0.1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    ob, lb = brute.brute_sparse_decode(q.tolist(), [{k: v.tolist() for k, v in dict(p, slots=past).items()}],
                                       0.1, 1.0, None)
    np.testing.assert_allclose(o1, np.array(ob), rtol=0, atol=1e-12)
