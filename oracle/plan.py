"""Occupancy-pinned split-KV plan (integer algorithm).

Test infrastructure only (see ``oracle/__init__``).

[T5] module docstring ("Split-KV scheduling is occupancy-pinned") and
``plan_split_kv`` / ``SplitPlan``. In units of 128-key tiles:
  * tiles_b = max(1, ceil(L_b / 128)), T = max_b tiles_b
  * one wave of the (work items, q-row tiles, kv heads) grid holds
    slots = max(1, cu_count * wg_per_cu // (h_k * n_q_tiles)) work items
  * lo = max(min_chunk_tiles, ceil(T / max_splits)) caps chunks per sequence
  * chunk = max(lo, ceil(T / force_splits)) when force_splits > 0;
    else chunk = T when the batch alone fills the wave (num_seqs >= slots)
    or max_splits == 1; else the smallest chunk >= lo whose chunk count
    sum_b ceil(tiles_b / chunk) fits in ``slots``
  * sequence b becomes work items (b, j*chunk, min((j+1)*chunk, tiles_b), j)
    for j < ceil(tiles_b / chunk); n_splits[b] is that count
  * work items are ordered longest first, ties keeping their order
  * pad_to > 0 appends empty items (0, 0, 0, 0) up to pad_to entries.

Errors (ValueError) where the page's asserts fire: pad_to below the number of
work items, more chunks than max_splits. Also rejected here: an empty batch,
negative lengths, non-positive sizes (the page never passes them).

The chunk is found by a plain upward scan from lo (the library bisects).

Pinned by tests/test_plan_oracle.py: hand-worked examples, the minimality of
the chunk (it fits, one tile less does not), coverage/contiguity of every
sequence's chunks, the wave bound, the ordering and the padding.
"""

import bisect

TILE_KEYS = 128


def _ceil_div(a, b):
    return -(-a // b)


def plan_split_kv(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16, force_splits=0,
                  min_chunk_tiles=1, pad_to=0):
    """Returns (work list of (seq, tile_begin, tile_end, split_slot), n_splits
    per sequence, chunk_tiles, slots)."""
    seq_lens = [int(x) for x in seq_lens]
    if not seq_lens:
        raise ValueError("empty batch")
    if any(x < 0 for x in seq_lens):
        raise ValueError("negative sequence length")
    if min(h_k, n_q_tiles, cu_count, wg_per_cu, max_splits, min_chunk_tiles) < 1:
        raise ValueError("sizes must be positive")
    if force_splits < 0 or pad_to < 0:
        raise ValueError("force_splits and pad_to must be >= 0")

    tiles = [max(1, _ceil_div(L, TILE_KEYS)) for L in seq_lens]
    t_max = max(tiles)
    slots = max(1, (cu_count * wg_per_cu) // (h_k * n_q_tiles))
    lo = max(min_chunk_tiles, _ceil_div(t_max, max_splits))

    def fits_one_wave(chunk):
        return sum(_ceil_div(t, chunk) for t in tiles) <= slots

    if force_splits > 0:
        chunk = max(lo, _ceil_div(t_max, force_splits))
    elif len(tiles) >= slots or max_splits == 1:
        chunk = t_max
    else:
        # scan upward from lo for the first chunk size that fits; t_max fits
        # (one chunk per sequence, fewer sequences than slots), and when lo
        # already exceeds t_max the chunk is lo
        chunk = next((c for c in range(lo, t_max + 1) if fits_one_wave(c)), lo)

    items = []  # (seq, first tile, end tile, split slot) in construction order
    n_splits = []
    for b, t in enumerate(tiles):
        cuts = list(range(0, t, chunk)) + [t]
        n_splits.append(len(cuts) - 1)
        for slot, (first, end) in enumerate(zip(cuts[:-1], cuts[1:])):
            items.append((b, first, end, slot))
    if max(n_splits) > max_splits:
        raise ValueError(f"{max(n_splits)} chunks exceed max_splits={max_splits}")
    # longest first; equal lengths keep construction order
    order = sorted(range(len(items)), key=lambda i: (items[i][1] - items[i][2], i))
    work = [items[i] for i in order]
    if pad_to:
        if pad_to < len(work):
            raise ValueError(f"pad_to {pad_to} < {len(work)} work items")
        work.extend([(0, 0, 0, 0)] * (pad_to - len(work)))
    return work, n_splits, chunk, slots


BALANCE_BLOCK_KEYS = 32


def plan_balanced(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16):
    """Balanced contiguous plan (the library's own planner, not the pages'):
    the 32-key blocks of all sequences (max(1, ceil(L / 32)) each), laid end
    to end in sequence order, are cut into `bins` contiguous shares of
    floor/ceil(total / bins) blocks, bins = the workgroups that run at once
    (the ``slots`` of the rule above). Bin i takes global blocks
    [floor(i * total / bins), floor((i+1) * total / bins)); every (sequence,
    share) overlap is a work item (seq, key_begin, key_end, slot) in keys:
    key_begin = 32 * its first block, key_end = min(32 * its end block, L),
    split slots numbered in key order. If some sequence would be cut into more
    than max_splits pieces, bins is lowered until none is. Returns (work
    ordered by bin, n_splits, bin_offsets[bins + 1], bins).
    """
    seq_lens = [int(x) for x in seq_lens]
    if not seq_lens:
        raise ValueError("empty batch")
    if any(x < 0 for x in seq_lens):
        raise ValueError("negative sequence length")
    if min(h_k, n_q_tiles, cu_count, wg_per_cu, max_splits) < 1:
        raise ValueError("sizes must be positive")
    blocks = [max(1, _ceil_div(L, BALANCE_BLOCK_KEYS)) for L in seq_lens]
    total = sum(blocks)
    starts = [0]
    for t in blocks:
        starts.append(starts[-1] + t)
    bins = max(1, min(total, (cu_count * wg_per_cu) // (h_k * n_q_tiles)))

    def pieces_for(nb):
        """Shares that overlap each sequence when `total` blocks are cut into nb."""
        bounds = [(i * total) // nb for i in range(nb + 1)]
        # share holding global block x: the last i with bounds[i] <= x
        share = lambda x: bisect.bisect_right(bounds, x) - 1  # noqa: E731
        return [share(starts[b + 1] - 1) - share(starts[b]) + 1 for b in range(len(blocks))], bounds

    while True:
        pieces, bounds = pieces_for(bins)
        if max(pieces) <= max_splits or bins == 1:
            break
        bins -= 1
    if max(pieces) > max_splits:
        raise ValueError(f"{max(pieces)} chunks exceed max_splits={max_splits}")
    work, offsets, seen = [], [0], [0] * len(blocks)
    for i in range(bins):
        lo, hi = bounds[i], bounds[i + 1]
        for b in range(len(blocks)):
            first, end = max(lo, starts[b]) - starts[b], min(hi, starts[b + 1]) - starts[b]
            if first < end:
                work.append((b, BALANCE_BLOCK_KEYS * first, min(BALANCE_BLOCK_KEYS * end, seq_lens[b]), seen[b]))
                seen[b] += 1
        offsets.append(len(work))
    return work, pieces, offsets, bins


def plan_queued(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16, pieces_per_bin=3, dyn_percent=10):
    """Queued plan (the library's own planner, not the pages'), written out step
    by step:
      1. blocks_b = max(1, ceil(L_b / 32)); total = sum; bins = the slots of
         the rule above, at most total;
      2. piece = max(1, total // (bins * pieces_per_bin)),
         budget = total * (100 - dyn_percent) // (100 * bins);
      3. sequence b is cut into n_b = ceil(blocks_b / max(piece,
         ceil(blocks_b / max_splits))) pieces, piece j covering blocks
         [j * blocks_b // n_b, (j + 1) * blocks_b // n_b), split slot j;
      4. pieces, longest first (ties: sequence, then piece), each go to the
         least loaded bin (lowest index among equals);
      5. bins in order hand their most recently assigned piece to the queue
         while they hold more than one piece and their load exceeds budget;
      6. the queue keeps the order of step 4.
    Work items (seq, 32 * first block, 32 * end block, slot) are listed bin
    by bin, then the queue. Returns (work, n_splits, bin_offsets[bins + 1],
    bins, queue length)."""
    seq_lens = [int(x) for x in seq_lens]
    if not seq_lens:
        raise ValueError("empty batch")
    if any(x < 0 for x in seq_lens):
        raise ValueError("negative sequence length")
    if min(h_k, n_q_tiles, cu_count, wg_per_cu, max_splits, pieces_per_bin) < 1:
        raise ValueError("sizes must be positive")
    if not 0 <= dyn_percent <= 90:
        raise ValueError("dyn_percent outside [0, 90]")
    blocks = [max(1, _ceil_div(L, BALANCE_BLOCK_KEYS)) for L in seq_lens]
    total = sum(blocks)
    bins = max(1, min(total, (cu_count * wg_per_cu) // (h_k * n_q_tiles)))
    piece = max(1, total // (bins * pieces_per_bin))
    budget = total * (100 - dyn_percent) // (100 * bins)

    pieces, n_splits = [], []
    for b, bl in enumerate(blocks):
        n = _ceil_div(bl, max(piece, _ceil_div(bl, max_splits)))
        n_splits.append(n)
        pieces.extend((b, j * bl // n, (j + 1) * bl // n, j) for j in range(n))
    order = sorted(range(len(pieces)), key=lambda i: (-(pieces[i][2] - pieces[i][1]), i))
    loads = [0] * bins
    members = [[] for _ in range(bins)]
    for i in order:
        k = min(range(bins), key=lambda x: (loads[x], x))
        loads[k] += pieces[i][2] - pieces[i][1]
        members[k].append(i)
    rank = {i: r for r, i in enumerate(order)}
    queue = []
    for k in range(bins):
        while len(members[k]) > 1 and loads[k] > budget:
            i = members[k].pop()
            loads[k] -= pieces[i][2] - pieces[i][1]
            queue.append(i)
    queue.sort(key=lambda i: rank[i])

    def item(i):
        b, first, end, slot = pieces[i]
        return (b, BALANCE_BLOCK_KEYS * first, BALANCE_BLOCK_KEYS * end, slot)

    work, offsets = [], [0]
    for k in range(bins):
        work.extend(item(i) for i in members[k])
        offsets.append(len(work))
    work.extend(item(i) for i in queue)
    return work, n_splits, offsets, bins, len(queue)


def plan_even(seq_lens, h_k, n_q_tiles, cu_count, wg_per_cu=1, max_splits=16):
    """The library's even plan: the occupancy-pinned rule at 32-key
    granularity (blocks of 32 keys instead of 128-key tiles), each sequence
    cut into pieces whose block counts differ by at most one. Returns (work
    list of (seq, key_begin, key_end, split_slot) in keys, longest first,
    n_splits, c in blocks, slots). A plain scan over c, not a bisection."""
    seq_lens = [int(x) for x in seq_lens]
    if not seq_lens:
        raise ValueError("empty batch")
    if any(x < 0 for x in seq_lens):
        raise ValueError("negative sequence length")
    if min(h_k, n_q_tiles, cu_count, wg_per_cu, max_splits) < 1:
        raise ValueError("sizes must be positive")
    blocks = [max(1, _ceil_div(L, BALANCE_BLOCK_KEYS)) for L in seq_lens]
    slots = max(1, (cu_count * wg_per_cu) // (h_k * n_q_tiles))
    b_max = max(blocks)
    c = b_max
    if len(blocks) < slots and max_splits > 1:
        for cand in range(_ceil_div(b_max, max_splits), b_max + 1):
            if sum(_ceil_div(x, cand) for x in blocks) <= slots:
                c = cand
                break
    work, n_splits = [], []
    for b, x in enumerate(blocks):
        k = _ceil_div(x, c)
        n_splits.append(k)
        cuts = [j * x // k for j in range(k + 1)]
        work.extend((b, BALANCE_BLOCK_KEYS * cuts[j], BALANCE_BLOCK_KEYS * cuts[j + 1], j) for j in range(k))
    work.sort(key=lambda w: w[1] - w[2])  # longest first; sort is stable
    return work, n_splits, c, slots


def plan_paired(seq_lens, pair_slots, max_splits=16):
    """Paired plan (the library's own planner, not the pages'): the chunks of
    the occupancy-pinned rule above, two per workgroup. For a candidate chunk
    c (in 128-key tiles), sequence b becomes ceil(tiles_b / c) pieces of c
    tiles (the last one shorter). The pieces are ranked longest first (equal
    lengths in construction order: sequence, then piece) and the ranking is
    padded with empty items to 2 * pair_slots places; workgroup k gets places
    k and 2 * pair_slots - 1 - k. The chunk is the first c counting up from
    ceil(T / max_splits) for which the pieces fit the places and no
    workgroup gets more than c tiles. Returns (work as a flat list of
    2 * min(pair_slots, n) items (seq, tile_begin, tile_end, split_slot),
    the two items of workgroup k at 2k and 2k + 1; n_splits; chunk)."""
    seq_lens = [int(x) for x in seq_lens]
    if not seq_lens:
        raise ValueError("empty batch")
    if any(x < 0 for x in seq_lens):
        raise ValueError("negative sequence length")
    if min(pair_slots, max_splits) < 1:
        raise ValueError("sizes must be positive")
    tiles = [max(1, _ceil_div(L, TILE_KEYS)) for L in seq_lens]
    places = 2 * pair_slots
    size = lambda item: item[2] - item[1]  # noqa: E731
    for chunk in range(_ceil_div(max(tiles), max_splits), max(tiles) + 1):
        pieces = [(b, s, min(s + chunk, t), j)
                  for b, t in enumerate(tiles) for j, s in enumerate(range(0, t, chunk))]
        if len(pieces) > places:
            continue
        ranked = [p for _, p in sorted(enumerate(pieces), key=lambda ip: (-size(ip[1]), ip[0]))]
        ranked += [(0, 0, 0, 0)] * (places - len(ranked))
        if all(size(ranked[k]) + size(ranked[places - 1 - k]) <= chunk for k in range(pair_slots)):
            break
    else:
        raise ValueError("no chunk puts the batch into pairs of at most one chunk")
    work = []
    for k in range(min(pair_slots, len(pieces))):
        work += [ranked[k], ranked[places - 1 - k]]
    return work, [_ceil_div(t, chunk) for t in tiles], chunk
