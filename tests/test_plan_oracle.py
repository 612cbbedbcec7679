"""Pins of the split-KV plan oracle (no GPU): hand-worked examples of the
rule on the t5_decode page (``plan_split_kv``), the chunk's minimality (it
fits one wave, one tile less does not), and the structural invariants of
every plan."""

import math

import numpy as np
import pytest

from oracle.plan import plan_split_kv


def test_hand_worked_split():
    # tiles [3, 8, 2, 1], slots = 5*2 // 2 = 5, lo = 1.
    # chunk 1 -> 14 items, 2 -> 8, 3 -> 6, 4 -> 5 <= 5: chunk = 4.
    work, ns, chunk, slots = plan_split_kv([300, 1000, 129, 50], h_k=2, n_q_tiles=1, cu_count=5, wg_per_cu=2)
    assert (chunk, slots, ns) == (4, 5, [1, 2, 1, 1])
    assert work == [(1, 0, 4, 0), (1, 4, 8, 1), (0, 0, 3, 0), (2, 0, 2, 0), (3, 0, 1, 0)]


def test_hand_worked_batch_fills_wave():
    # slots = 4 // 4 = 1 <= 8 sequences: nothing is split.
    work, ns, chunk, slots = plan_split_kv([5000] * 8, h_k=4, n_q_tiles=1, cu_count=4, wg_per_cu=1)
    assert (chunk, slots) == (40, 1)
    assert work == [(b, 0, 40, 0) for b in range(8)] and ns == [1] * 8


def test_hand_worked_force_splits_and_stable_order():
    # tiles [8, 2]; chunk = max(1, ceil(8 / 3)) = 3.
    work, ns, chunk, _ = plan_split_kv([1000, 200], h_k=1, n_q_tiles=1, cu_count=64, force_splits=3)
    assert chunk == 3 and ns == [3, 1]
    assert work == [(0, 0, 3, 0), (0, 3, 6, 1), (0, 6, 8, 2), (1, 0, 2, 0)]


def test_hand_worked_max_splits_cap():
    # tiles [64, 1]; lo = ceil(64 / 16) = 4 and 4 already fits 1024 slots.
    work, ns, chunk, slots = plan_split_kv([128 * 64, 128], h_k=1, n_q_tiles=1, cu_count=256, wg_per_cu=4)
    assert (chunk, slots, ns) == (4, 1024, [16, 1])
    assert len(work) == 17 and work[-1] == (1, 0, 1, 0)


def test_hand_worked_single_split_and_empty_sequence():
    work, ns, chunk, _ = plan_split_kv([0, 130, 37], h_k=1, n_q_tiles=1, cu_count=256, max_splits=1)
    assert chunk == 2 and ns == [1, 1, 1]
    assert work == [(1, 0, 2, 0), (0, 0, 1, 0), (2, 0, 1, 0)]


def test_padding_and_errors():
    work, *_ = plan_split_kv([300, 1000, 129, 50], h_k=2, n_q_tiles=1, cu_count=5, wg_per_cu=2, pad_to=8)
    assert work[5:] == [(0, 0, 0, 0)] * 3 and len(work) == 8
    with pytest.raises(ValueError):
        plan_split_kv([300, 1000, 129, 50], h_k=2, n_q_tiles=1, cu_count=5, wg_per_cu=2, pad_to=4)
    with pytest.raises(ValueError):
        plan_split_kv([], h_k=1, n_q_tiles=1, cu_count=1)
    with pytest.raises(ValueError):
        plan_split_kv([-1], h_k=1, n_q_tiles=1, cu_count=1)
    with pytest.raises(ValueError):
        plan_split_kv([10], h_k=0, n_q_tiles=1, cu_count=1)


def _check_invariants(lens, kw, work, ns, chunk, slots):
    tiles = [max(1, math.ceil(L / 128)) for L in lens]
    real = [w for w in work if w[2] > w[1]]
    per_seq = {}
    for w in real:
        per_seq.setdefault(w[0], []).append(w)
    for b, t in enumerate(tiles):
        items = sorted(per_seq[b], key=lambda w: w[3])
        assert [w[3] for w in items] == list(range(ns[b]))
        assert items[0][1] == 0 and items[-1][2] == t
        for a, c in zip(items, items[1:]):
            assert a[2] == c[1]
        assert all(w[2] - w[1] <= chunk for w in items)
    assert max(ns) <= kw.get("max_splits", 16)
    lengths = [w[2] - w[1] for w in real]
    assert lengths == sorted(lengths, reverse=True)
    assert all(w == (0, 0, 0, 0) for w in work[len(real):])
    # ties keep generation order (sequence-major, split-slot minor)
    for a, c in zip(real, real[1:]):
        if a[2] - a[1] == c[2] - c[1]:
            assert (a[0], a[3]) < (c[0], c[3])


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_invariants_and_minimal_chunk(seed):
    rng = np.random.default_rng(seed)
    b = int(rng.integers(1, 80))
    lens = rng.integers(0, 70000, size=b).tolist()
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 17)), max_splits=int(rng.choice([1, 4, 16, 64])),
              min_chunk_tiles=int(rng.choice([1, 1, 2, 8])))
    work, ns, chunk, slots = plan_split_kv(lens, **kw)
    _check_invariants(lens, kw, work, ns, chunk, slots)
    tiles = [max(1, math.ceil(L / 128)) for L in lens]
    assert slots == max(1, 256 * kw["wg_per_cu"] // (kw["h_k"] * kw["n_q_tiles"]))
    lo = max(kw["min_chunk_tiles"], math.ceil(max(tiles) / kw["max_splits"]))
    if len(tiles) >= slots or kw["max_splits"] == 1:
        assert chunk == max(tiles)
    else:
        # minimal: the chunk fits one wave and one tile less (when still >= lo) does not; the chunk count
        # only grows as the chunk shrinks, so no smaller size fits either
        def count(c):
            return sum(math.ceil(t / c) for t in tiles)
        assert chunk >= lo and (count(chunk) <= slots or chunk == lo > max(tiles))
        assert chunk == lo or count(chunk - 1) > slots


# ---------------------------------------------------------------------------
# balanced contiguous plan (the build's own planner)
# ---------------------------------------------------------------------------
from oracle.plan import plan_balanced  # noqa: E402


def test_balanced_hand_worked():
    # 32-key blocks [10, 32, 5, 2], 49 in total, starting at 0, 10, 42, 47; slots = 5*2 // 2 = 5 bins,
    # cut at 49*i // 5 = 0, 9, 19, 29, 39, 49
    work, ns, off, bins = plan_balanced([300, 1000, 129, 50], h_k=2, n_q_tiles=1, cu_count=5, wg_per_cu=2)
    assert bins == 5
    assert work == [(0, 0, 288, 0),                      # bin 0: global blocks [0, 9)
                    (0, 288, 300, 1), (1, 0, 288, 0),    # bin 1: [9, 19), sequence 0 ends at L = 300
                    (1, 288, 608, 1),                    # bin 2: [19, 29)
                    (1, 608, 928, 2),                    # bin 3: [29, 39)
                    (1, 928, 1000, 3), (2, 0, 129, 0), (3, 0, 50, 0)]  # bin 4: [39, 49)
    assert off == [0, 1, 3, 4, 5, 8] and ns == [2, 4, 1, 1]


def test_balanced_lowers_bins_for_max_splits():
    # one sequence of 256 blocks over 32 bins would be 32 pieces; max_splits 8 -> 8 bins of 1024 keys
    work, ns, off, bins = plan_balanced([64 * 128], h_k=1, n_q_tiles=1, cu_count=32, max_splits=8)
    assert bins == 8 and ns == [8]
    assert [w[2] - w[1] for w in work] == [1024] * 8


def test_balanced_empty_sequence_is_one_block():
    # L = 0 still takes one block, so its (empty) item exists and its output gets written
    work, ns, off, bins = plan_balanced([0, 64], h_k=1, n_q_tiles=1, cu_count=3)
    assert bins == 3 and work == [(0, 0, 0, 0), (1, 0, 32, 0), (1, 32, 64, 1)] and ns == [1, 2]
    assert off == [0, 1, 2, 3]


@pytest.mark.parametrize("seed", range(40))
def test_balanced_invariants(seed):
    rng = np.random.default_rng(5000 + seed)
    b = int(rng.integers(1, 100))
    lens = rng.integers(0, 70000, size=b)
    lens[rng.random(b) < 0.1] = 0
    lens = lens.tolist()
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([4, 16, 64, 256])))
    work, ns, off, bins = plan_balanced(lens, **kw)
    blocks = [max(1, math.ceil(L / 32)) for L in lens]
    total = sum(blocks)
    assert len(off) == bins + 1 and off[0] == 0 and off[-1] == len(work)

    def nblk(w):
        return 1 if lens[w[0]] == 0 else math.ceil(w[2] / 32) - w[1] // 32

    # every bin holds floor or ceil of total / bins blocks, contiguous in sequence order
    loads = [sum(nblk(w) for w in work[off[i]:off[i + 1]]) for i in range(bins)]
    assert sum(loads) == total and max(loads) - min(loads) <= 1
    # the items of a sequence tile [0, L) in key order, cut at multiples of 32
    for s in range(len(lens)):
        items = [w for w in work if w[0] == s]
        assert items[0][1] == 0 and items[-1][2] == lens[s]
        assert all(a[2] == c[1] for a, c in zip(items, items[1:]))
        assert all(w[1] % 32 == 0 and (w[2] % 32 == 0 or w[2] == lens[s]) for w in items)
        assert all(w[2] > w[1] for w in items) or lens[s] == 0
        # split slots count up per sequence; n_splits matches
        assert [w[3] for w in items] == list(range(len(items))) and ns[s] == len(items)
    # items appear in global order (bin by bin, sequence order inside a bin)
    assert [(w[0], w[1]) for w in work] == sorted((w[0], w[1]) for w in work)
    assert max(ns) <= kw["max_splits"]
    assert bins <= max(1, 256 * kw["wg_per_cu"] // (kw["h_k"] * kw["n_q_tiles"]))


# ---------------------------------------------------------------------------
# queued plan (the build's own planner): packed bins, then a shared queue
# ---------------------------------------------------------------------------
from oracle.plan import plan_queued  # noqa: E402


def test_queued_hand_worked():
    # blocks [10, 4, 1] (15), bins = 3, piece = 15 // (3 * 2) = 2, budget = 15 * 80 // 300 = 4.
    # pieces: seq 0 -> five of 2 blocks, seq 1 -> two of 2, seq 2 -> one of 1; longest first in input order.
    # least loaded bin: s0p0 b0, s0p1 b1, s0p2 b2, s0p3 b0, s0p4 b1, s1p0 b2, s1p1 b0 (6), s2p0 b1 (5).
    # over budget: bin 0 gives s1p1, bin 1 gives s2p0; the queue keeps longest-first order.
    work, ns, off, bins, nq = plan_queued([300, 100, 0], h_k=1, n_q_tiles=1, cu_count=3, pieces_per_bin=2,
                                          dyn_percent=20)
    assert (bins, ns, off, nq) == (3, [5, 2, 1], [0, 2, 4, 6], 2)
    assert work == [(0, 0, 64, 0), (0, 192, 256, 3),      # bin 0
                    (0, 64, 128, 1), (0, 256, 320, 4),    # bin 1
                    (0, 128, 192, 2), (1, 0, 64, 0),      # bin 2
                    (1, 64, 128, 1), (2, 0, 32, 0)]       # queue


def test_queued_small_exact():
    # two sequences, blocks [4, 2], bins = 2, piece = 6 // 2 = 3, budget = 6*50 // 200 = 1:
    # seq 0 -> 2 pieces [0,2) [2,4), seq 1 -> 1 piece [0,2); all of size 2, longest-first keeps input order.
    # bins: (0,0,2)->0, (0,2,4)->1, (1,0,2)->0; bin 0 is over budget with 2 pieces -> (1,0,2) queued.
    work, ns, off, bins, nq = plan_queued([128, 64], h_k=1, n_q_tiles=1, cu_count=2, pieces_per_bin=1,
                                          dyn_percent=50)
    assert (bins, ns, off, nq) == (2, [2, 1], [0, 1, 2], 1)
    assert work == [(0, 0, 64, 0), (0, 64, 128, 1), (1, 0, 64, 0)]


def test_queued_errors():
    with pytest.raises(ValueError):
        plan_queued([10], h_k=1, n_q_tiles=1, cu_count=1, pieces_per_bin=0)
    with pytest.raises(ValueError):
        plan_queued([10], h_k=1, n_q_tiles=1, cu_count=1, dyn_percent=95)
    with pytest.raises(ValueError):
        plan_queued([], h_k=1, n_q_tiles=1, cu_count=1)


@pytest.mark.parametrize("seed", range(30))
def test_queued_invariants(seed):
    rng = np.random.default_rng(7000 + seed)
    b = int(rng.integers(1, 90))
    lens = rng.integers(0, 70000, size=b)
    lens[rng.random(b) < 0.1] = 0
    lens = lens.tolist()
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=int(rng.choice([8, 64, 256])),
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([4, 16, 64, 256])),
              pieces_per_bin=int(rng.integers(1, 5)), dyn_percent=int(rng.integers(0, 60)))
    work, ns, off, bins, nq = plan_queued(lens, **kw)
    blocks = [max(1, math.ceil(L / 32)) for L in lens]
    total = sum(blocks)
    budget = total * (100 - kw["dyn_percent"]) // (100 * bins)
    assert len(off) == bins + 1 and off[0] == 0 and off[-1] + nq == len(work)
    size = lambda w: (w[2] - w[1]) // 32  # noqa: E731
    for i in range(bins):
        members = work[off[i]:off[i + 1]]  # may be empty when max_splits makes pieces few and large
        assert sum(size(w) for w in members) <= budget or len(members) == 1
    queue = work[off[-1]:]
    assert [size(w) for w in queue] == sorted((size(w) for w in queue), reverse=True)
    for s in range(len(lens)):
        items = sorted(w for w in work if w[0] == s)
        assert items[0][1] == 0 and items[-1][2] == 32 * blocks[s]
        assert all(a[2] == c[1] for a, c in zip(items, items[1:]))
        assert [w[3] for w in items] == list(range(len(items))) and ns[s] == len(items)
        assert max(size(w) for w in items) - min(size(w) for w in items) <= 1  # even cut
    assert max(ns) <= kw["max_splits"]


from oracle.plan import plan_even, plan_split_kv as _tile_plan  # noqa: E402


def test_even_hand_worked():
    # blocks of 32 keys: [10, 4, 1], 4 slots; c = 1..4 give 15, 8, 7, 5 pieces,
    # c = 5 gives 2 + 1 + 1 = 4
    work, ns, c, slots = plan_even([300, 100, 0], h_k=1, n_q_tiles=1, cu_count=4)
    assert (c, slots, ns) == (5, 4, [2, 1, 1])
    assert work == [(0, 0, 160, 0), (0, 160, 320, 1), (1, 0, 128, 0), (2, 0, 32, 0)]


def test_even_unequal_pieces_differ_by_one_block():
    # 7 blocks in 3 pieces: cuts at 7*1//3 = 2 and 7*2//3 = 4 -> 2, 2, 3 blocks
    work, ns, c, slots = plan_even([224], h_k=1, n_q_tiles=1, cu_count=3)
    assert c == 3 and ns == [3]
    assert work == [(0, 128, 224, 2), (0, 0, 64, 0), (0, 64, 128, 1)]


def test_even_errors():
    with pytest.raises(ValueError):
        plan_even([], h_k=1, n_q_tiles=1, cu_count=1)
    with pytest.raises(ValueError):
        plan_even([-1], h_k=1, n_q_tiles=1, cu_count=1)
    with pytest.raises(ValueError):
        plan_even([10], h_k=0, n_q_tiles=1, cu_count=1)


@pytest.mark.parametrize("seed", range(12))
def test_even_invariants(seed):
    rng = np.random.default_rng(700 + seed)
    n = int(rng.integers(1, 90))
    lens = rng.integers(0, 20000, size=n).tolist()
    kw = dict(h_k=int(rng.choice([1, 2, 4, 8])), n_q_tiles=int(rng.integers(1, 3)), cu_count=256,
              wg_per_cu=int(rng.integers(1, 9)), max_splits=int(rng.choice([1, 4, 16, 64])))
    work, ns, c, slots = plan_even(lens, **kw)
    if len(lens) < slots and kw["max_splits"] > 1:
        assert len(work) <= slots
    lengths = [w[2] - w[1] for w in work]
    assert lengths == sorted(lengths, reverse=True)
    for b, L in enumerate(lens):
        mine = sorted((w for w in work if w[0] == b), key=lambda w: w[1])
        assert len(mine) == ns[b] <= kw["max_splits"]
        assert [w[3] for w in mine] == list(range(ns[b]))
        assert mine[0][1] == 0 and mine[-1][2] == 32 * max(1, -(-L // 32))
        assert all(x[2] == y[1] for x, y in zip(mine, mine[1:]))  # contiguous cover
        assert all(w[1] % 32 == 0 and w[2] > w[1] for w in mine)
        sizes = [(w[2] - w[1]) // 32 for w in mine]
        assert max(sizes) - min(sizes) <= 1 and max(sizes) <= c
    # never a longer item than the 128-key tile plan of the same batch
    twork = _tile_plan(lens, **kw)[0]
    assert max(lengths) <= max((w[2] - w[1]) * 128 for w in twork)


from oracle.plan import plan_paired  # noqa: E402


def test_paired_hand_worked():
    # tiles [8, 1, 2, 4], three pairs. c = 4 fits five pieces into six places but
    # pairs the second 4-tile piece with the 1-tile one (5 > 4); c = 5 ranks
    # (seq 0 0-5) 5, (seq 3) 4, (seq 0 5-8) 3, (seq 2) 2, (seq 1) 1, pad:
    # pairs 5 + 0, 4 + 1, 3 + 2, all <= 5
    work, ns, chunk = plan_paired([1024, 100, 256, 512], pair_slots=3)
    assert chunk == 5 and ns == [2, 1, 1, 1]
    assert work == [(0, 0, 5, 0), (0, 0, 0, 0), (3, 0, 4, 0), (1, 0, 1, 0), (0, 5, 8, 1), (2, 0, 2, 0)]


def test_paired_fewer_items_than_pairs_and_errors():
    # tiles [3, 1], four pairs: c = 1 already fits (four one-tile pieces, each alone)
    work, ns, chunk = plan_paired([300, 100], pair_slots=4)
    assert chunk == 1 and ns == [3, 1]
    pad = (0, 0, 0, 0)
    assert work == [(0, 0, 1, 0), pad, (0, 1, 2, 1), pad, (0, 2, 3, 2), pad, (1, 0, 1, 0), pad]
    # max_splits = 1: c starts at the longest, one piece per sequence
    work, ns, chunk = plan_paired([300, 100], pair_slots=4, max_splits=1)
    assert chunk == 3 and ns == [1, 1] and work == [(0, 0, 3, 0), pad, (1, 0, 1, 0), pad]
    # max_splits caps the pieces: 8 tiles with max_splits 2 start at c = 4
    assert plan_paired([1024], pair_slots=4, max_splits=2)[2] == 4
    # five sequences of one tile in two pairs can never fit
    with pytest.raises(ValueError):
        plan_paired([128] * 5, pair_slots=2)
    # three sequences of 2 tiles in two pairs: a pair would hold 4 tiles > c = 2
    with pytest.raises(ValueError):
        plan_paired([256] * 3, pair_slots=2)
    for bad in ([], [-1]):
        with pytest.raises(ValueError):
            plan_paired(bad, pair_slots=2)
    with pytest.raises(ValueError):
        plan_paired([5], pair_slots=0)


@pytest.mark.parametrize("seed", range(40))
def test_paired_invariants_and_minimal_chunk(seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 40))
    lens = rng.integers(0, 9000, size=n).tolist()
    pair_slots = int(rng.integers(max(1, n // 2), 64))
    max_splits = int(rng.integers(1, 40))
    try:
        work, ns, chunk = plan_paired(lens, pair_slots, max_splits)
    except ValueError:
        return
    tiles = [max(1, math.ceil(L / 128)) for L in lens]
    real = [w for w in work if w[2] > w[1]]
    # coverage: every sequence's tiles exactly once, pieces of `chunk` tiles in order, split slots 0..k-1
    for b, t in enumerate(tiles):
        mine = sorted((w for w in real if w[0] == b), key=lambda w: w[1])
        assert [w[3] for w in mine] == list(range(len(mine))) == list(range(ns[b]))
        assert mine[0][1] == 0 and mine[-1][2] == t
        assert all(x[2] == y[1] for x, y in zip(mine, mine[1:]))
        assert all(w[2] - w[1] == chunk for w in mine[:-1]) and 0 < mine[-1][2] - mine[-1][1] <= chunk
    assert max(ns) <= max_splits and len(work) == 2 * min(pair_slots, len(real))
    # the first items of the pairs are the longest, in order; no pair above one chunk
    firsts = [work[2 * k][2] - work[2 * k][1] for k in range(len(work) // 2)]
    assert firsts == sorted(firsts, reverse=True)
    assert all((work[2 * k][2] - work[2 * k][1]) + (work[2 * k + 1][2] - work[2 * k + 1][1]) <= chunk
               for k in range(len(work) // 2))
    # minimality, by brute force over every smaller chunk: too many pieces, or some fold pair > c
    lo = math.ceil(max(tiles) / max_splits)
    assert chunk >= lo
    for c in range(lo, chunk):
        sizes = sorted((min(t, (j + 1) * c) - j * c for t in tiles for j in range(math.ceil(t / c))), reverse=True)
        if len(sizes) > 2 * pair_slots:
            continue
        sizes += [0] * (2 * pair_slots - len(sizes))
        assert max(sizes[k] + sizes[-1 - k] for k in range(pair_slots)) > c
