// Occupancy-pinned split-KV planner (host only).
//
// Rule of "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", plan_split_kv
// and its module docstring ("Split-KV scheduling is occupancy-pinned"): pick
// the smallest contiguous chunk of 128-key tiles such that the chunks of all
// sequences fit one wave of workgroup slots, capped at max_splits chunks per
// sequence; emit one work item per chunk, longest first.
#include <algorithm>
#include <cstdint>
#include <vector>

#include "pkv_internal.h"

namespace {

constexpr int64_t kTileKeys = 128;
constexpr int64_t kBalanceBlockKeys = 32;  // cut granularity of the balanced plan

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Item {
  int32_t seq, begin, end, slot;
};

}  // namespace

extern "C" pkv_status pkv_plan_split_kv(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                                        int32_t cu_count, int32_t wg_per_cu, int32_t max_splits,
                                        int32_t force_splits, int32_t min_chunk_tiles, int32_t pad_to,
                                        int32_t* work_out, int32_t work_cap, int32_t* n_splits_out,
                                        pkv_plan_info* info) {
  using pkv::fail;
  if (!seq_lens || !work_out || !n_splits_out) return fail(PKV_ERR_INVALID_ARG, "plan: NULL array");
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "plan: num_seqs=%d < 1", num_seqs);
  if (h_k < 1 || n_q_tiles < 1 || cu_count < 1 || wg_per_cu < 1 || max_splits < 1 || min_chunk_tiles < 1)
    return fail(PKV_ERR_INVALID_ARG, "plan: sizes must be >= 1 (h_k=%d n_q_tiles=%d cu=%d wg/cu=%d max_splits=%d "
                "min_chunk=%d)", h_k, n_q_tiles, cu_count, wg_per_cu, max_splits, min_chunk_tiles);
  if (force_splits < 0 || pad_to < 0 || work_cap < 0)
    return fail(PKV_ERR_INVALID_ARG, "plan: force_splits, pad_to and work_cap must be >= 0");
  if (max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_UNSUPPORTED, "plan: max_splits=%d > %d", max_splits, PKV_MAX_SPLITS);

  std::vector<int64_t> tiles(num_seqs);
  int64_t t_max = 1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    tiles[b] = std::max<int64_t>(1, ceil_div(seq_lens[b], kTileKeys));
    t_max = std::max(t_max, tiles[b]);
  }
  const int64_t slots = std::max<int64_t>(1, ((int64_t)cu_count * wg_per_cu) / ((int64_t)h_k * n_q_tiles));
  const int64_t lo = std::max<int64_t>(min_chunk_tiles, ceil_div(t_max, max_splits));
  auto n_chunks = [&](int64_t c) {
    int64_t s = 0;
    for (int64_t t : tiles) s += ceil_div(t, c);
    return s;
  };

  int64_t chunk;
  if (force_splits > 0) {
    chunk = std::max(lo, ceil_div(t_max, force_splits));
  } else if (num_seqs >= slots || max_splits == 1) {
    chunk = t_max;
  } else {
    // n_chunks is non-increasing in c and t_max always fits (one chunk per
    // sequence, num_seqs < slots): bisect for the smallest fitting c.
    int64_t a = lo, z = t_max;
    while (a < z) {
      const int64_t mid = a + (z - a) / 2;
      if (n_chunks(mid) <= slots)
        z = mid;
      else
        a = mid + 1;
    }
    chunk = a;
  }

  std::vector<Item> items;
  int32_t max_ns = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t k = ceil_div(tiles[b], chunk);
    if (k > max_splits)
      return fail(PKV_ERR_UNSUPPORTED, "plan: sequence %d needs %lld chunks > max_splits=%d", b, (long long)k,
                  max_splits);
    n_splits_out[b] = (int32_t)k;
    max_ns = std::max<int32_t>(max_ns, (int32_t)k);
    for (int64_t j = 0; j < k; ++j)
      items.push_back({b, (int32_t)(j * chunk), (int32_t)std::min((j + 1) * chunk, tiles[b]), (int32_t)j});
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& x, const Item& y) { return (x.end - x.begin) > (y.end - y.begin); });
  const int64_t n_real = (int64_t)items.size();
  if (pad_to && pad_to < n_real)
    return fail(PKV_ERR_CAPACITY, "plan: pad_to=%d < %lld work items", pad_to, (long long)n_real);
  const int64_t n_total = pad_to ? pad_to : n_real;
  if (n_total > work_cap)
    return fail(PKV_ERR_CAPACITY, "plan: %lld work items > work_cap=%d", (long long)n_total, work_cap);
  for (int64_t i = 0; i < n_total; ++i) {
    const Item it = i < n_real ? items[i] : Item{0, 0, 0, 0};
    work_out[4 * i + 0] = it.seq;
    work_out[4 * i + 1] = it.begin;
    work_out[4 * i + 2] = it.end;
    work_out[4 * i + 3] = it.slot;
  }
  if (info) {
    info->num_work = (int32_t)n_total;
    info->num_real = (int32_t)n_real;
    info->chunk_tiles = (int32_t)chunk;
    info->slots = (int32_t)std::min<int64_t>(slots, INT32_MAX);
    info->max_n_splits = max_ns;
    info->num_bins = 0;
    info->num_dynamic = 0;
  }
  return PKV_OK;
}

// Even plan (this library's own; see pkv_fp8.h): the rule above at 32-key
// granularity, each sequence cut into pieces as equal as 32-key blocks allow.
extern "C" pkv_status pkv_plan_even(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                                    int32_t cu_count, int32_t wg_per_cu, int32_t max_splits, int32_t* work_out,
                                    int32_t work_cap, int32_t* n_splits_out, pkv_plan_info* info) {
  using pkv::fail;
  if (!seq_lens || !work_out || !n_splits_out) return fail(PKV_ERR_INVALID_ARG, "plan: NULL array");
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "plan: num_seqs=%d < 1", num_seqs);
  if (h_k < 1 || n_q_tiles < 1 || cu_count < 1 || wg_per_cu < 1 || max_splits < 1)
    return fail(PKV_ERR_INVALID_ARG, "plan: sizes must be >= 1");
  if (work_cap < 0) return fail(PKV_ERR_INVALID_ARG, "plan: work_cap must be >= 0");
  if (max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_UNSUPPORTED, "plan: max_splits=%d > %d", max_splits, PKV_MAX_SPLITS);
  std::vector<int64_t> blocks(num_seqs);
  int64_t b_max = 1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    blocks[b] = std::max<int64_t>(1, ceil_div(seq_lens[b], kBalanceBlockKeys));
    b_max = std::max(b_max, blocks[b]);
  }
  const int64_t slots = std::max<int64_t>(1, ((int64_t)cu_count * wg_per_cu) / ((int64_t)h_k * n_q_tiles));
  const int64_t lo = ceil_div(b_max, max_splits);
  auto n_pieces = [&](int64_t c) {
    int64_t s = 0;
    for (int64_t x : blocks) s += ceil_div(x, c);
    return s;
  };
  int64_t c = b_max;
  if (num_seqs < slots && max_splits > 1) {
    int64_t a = lo, z = b_max;  // n_pieces is non-increasing in c; b_max always fits
    while (a < z) {
      const int64_t mid = a + (z - a) / 2;
      if (n_pieces(mid) <= slots)
        z = mid;
      else
        a = mid + 1;
    }
    c = a;
  }
  std::vector<Item> items;
  int32_t max_ns = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t k = ceil_div(blocks[b], c);  // <= max_splits since c >= lo
    n_splits_out[b] = (int32_t)k;
    max_ns = std::max<int32_t>(max_ns, (int32_t)k);
    for (int64_t j = 0; j < k; ++j)  // piece j: blocks [j * n / k, (j + 1) * n / k)
      items.push_back({b, (int32_t)(kBalanceBlockKeys * ((j * blocks[b]) / k)),
                       (int32_t)(kBalanceBlockKeys * (((j + 1) * blocks[b]) / k)), (int32_t)j});
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& x, const Item& y) { return (x.end - x.begin) > (y.end - y.begin); });
  const int64_t n = (int64_t)items.size();
  if (n > work_cap) return fail(PKV_ERR_CAPACITY, "plan: %lld work items > work_cap=%d", (long long)n, work_cap);
  for (int64_t i = 0; i < n; ++i) {
    work_out[4 * i + 0] = items[i].seq;
    work_out[4 * i + 1] = items[i].begin;
    work_out[4 * i + 2] = items[i].end;
    work_out[4 * i + 3] = items[i].slot;
  }
  if (info) {
    info->num_work = (int32_t)n;
    info->num_real = (int32_t)n;
    info->chunk_tiles = (int32_t)c;  // here in 32-key blocks
    info->slots = (int32_t)std::min<int64_t>(slots, INT32_MAX);
    info->max_n_splits = max_ns;
    info->num_bins = 0;
    info->num_dynamic = 0;
  }
  return PKV_OK;
}

// Balanced contiguous plan (this library's own; see pkv_fp8.h): tiles of all
// sequences end to end, cut into `bins` equal contiguous shares.
extern "C" pkv_status pkv_plan_balanced(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                                        int32_t cu_count, int32_t wg_per_cu, int32_t max_splits, int32_t* work_out,
                                        int32_t work_cap, int32_t* n_splits_out, int32_t* bin_offsets_out,
                                        int32_t bins_cap, pkv_plan_info* info) {
  using pkv::fail;
  if (!seq_lens || !work_out || !n_splits_out || !bin_offsets_out)
    return fail(PKV_ERR_INVALID_ARG, "plan: NULL array");
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "plan: num_seqs=%d < 1", num_seqs);
  if (h_k < 1 || n_q_tiles < 1 || cu_count < 1 || wg_per_cu < 1 || max_splits < 1)
    return fail(PKV_ERR_INVALID_ARG, "plan: sizes must be >= 1");
  if (work_cap < 0 || bins_cap < 0) return fail(PKV_ERR_INVALID_ARG, "plan: capacities must be >= 0");
  if (max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_UNSUPPORTED, "plan: max_splits=%d > %d", max_splits, PKV_MAX_SPLITS);
  std::vector<int64_t> start(num_seqs + 1, 0);
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    start[b + 1] = start[b] + std::max<int64_t>(1, ceil_div(seq_lens[b], kBalanceBlockKeys));
  }
  const int64_t total = start[num_seqs];
  int64_t bins = ((int64_t)cu_count * wg_per_cu) / ((int64_t)h_k * n_q_tiles);
  bins = std::max<int64_t>(1, std::min(bins, total));
  // share i covers global blocks [i*total/bins, (i+1)*total/bins); the share
  // holding block x is the last i with i*total/bins <= x
  auto share_of = [&](int64_t x, int64_t nb) {
    int64_t i = ((x + 1) * nb + total - 1) / total - 1;  // largest i with floor(i*total/nb) <= x
    while (i + 1 < nb && ((i + 1) * total) / nb <= x) ++i;
    while (i > 0 && (i * total) / nb > x) --i;
    return i;
  };
  auto max_pieces = [&](int64_t nb) {
    int64_t m = 0;
    for (int32_t b = 0; b < num_seqs; ++b) m = std::max(m, share_of(start[b + 1] - 1, nb) - share_of(start[b], nb) + 1);
    return m;
  };
  while (bins > 1 && max_pieces(bins) > max_splits) --bins;
  if (max_pieces(bins) > max_splits)
    return fail(PKV_ERR_UNSUPPORTED, "plan: a sequence needs more than max_splits=%d pieces", max_splits);
  if (bins + 1 > bins_cap) return fail(PKV_ERR_CAPACITY, "plan: %lld bins > bins_cap - 1", (long long)bins);

  std::vector<int32_t> seen(num_seqs, 0);
  int64_t n = 0;
  int32_t b = 0;
  bin_offsets_out[0] = 0;
  for (int64_t i = 0; i < bins; ++i) {
    const int64_t lo = (i * total) / bins, hi = ((i + 1) * total) / bins;
    while (b < num_seqs && start[b + 1] <= lo) ++b;
    for (int32_t c = b; c < num_seqs && start[c] < hi; ++c) {
      const int64_t s0 = std::max(lo, start[c]), e0 = std::min(hi, start[c + 1]);
      if (s0 >= e0) continue;
      if (n >= work_cap) return fail(PKV_ERR_CAPACITY, "plan: work items exceed work_cap=%d", work_cap);
      work_out[4 * n + 0] = c;
      work_out[4 * n + 1] = (int32_t)(kBalanceBlockKeys * (s0 - start[c]));
      work_out[4 * n + 2] = (int32_t)std::min<int64_t>(kBalanceBlockKeys * (e0 - start[c]), seq_lens[c]);
      work_out[4 * n + 3] = seen[c]++;
      ++n;
    }
    bin_offsets_out[i + 1] = (int32_t)n;
  }
  int32_t max_ns = 0;
  for (int32_t c = 0; c < num_seqs; ++c) {
    n_splits_out[c] = seen[c];
    max_ns = std::max(max_ns, seen[c]);
  }
  if (info) {
    info->num_work = (int32_t)n;
    info->num_real = (int32_t)n;
    info->chunk_tiles = (int32_t)ceil_div(ceil_div(total, bins), kTileKeys / kBalanceBlockKeys);
    info->slots = (int32_t)bins;
    info->max_n_splits = max_ns;
    info->num_bins = (int32_t)bins;
    info->num_dynamic = 0;
  }
  return PKV_OK;
}

// Queued plan (this library's own; see pkv_fp8.h): sequences cut into even
// pieces of 32-key blocks, packed longest first onto the least loaded of
// `bins` persistent workgroups; each bin then hands its last (smallest)
// pieces to a shared queue until its load fits the static budget, and the
// workgroups drain the queue as they finish.
extern "C" pkv_status pkv_plan_queued(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                                      int32_t cu_count, int32_t wg_per_cu, int32_t max_splits,
                                      int32_t pieces_per_bin, int32_t dyn_percent, int32_t* work_out,
                                      int32_t work_cap, int32_t* n_splits_out, int32_t* bin_offsets_out,
                                      int32_t bins_cap, pkv_plan_info* info) {
  using pkv::fail;
  if (!seq_lens || !work_out || !n_splits_out || !bin_offsets_out)
    return fail(PKV_ERR_INVALID_ARG, "plan: NULL array");
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "plan: num_seqs=%d < 1", num_seqs);
  if (h_k < 1 || n_q_tiles < 1 || cu_count < 1 || wg_per_cu < 1 || max_splits < 1 || pieces_per_bin < 1)
    return fail(PKV_ERR_INVALID_ARG, "plan: sizes must be >= 1");
  if (dyn_percent < 0 || dyn_percent > 90)
    return fail(PKV_ERR_INVALID_ARG, "plan: dyn_percent=%d not in [0, 90]", dyn_percent);
  if (work_cap < 0 || bins_cap < 0) return fail(PKV_ERR_INVALID_ARG, "plan: capacities must be >= 0");
  if (max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_UNSUPPORTED, "plan: max_splits=%d > %d", max_splits, PKV_MAX_SPLITS);
  std::vector<int64_t> blocks(num_seqs);
  int64_t total = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "plan: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    blocks[b] = std::max<int64_t>(1, ceil_div(seq_lens[b], kBalanceBlockKeys));
    total += blocks[b];
  }
  int64_t bins = ((int64_t)cu_count * wg_per_cu) / ((int64_t)h_k * n_q_tiles);
  bins = std::max<int64_t>(1, std::min(bins, total));
  if (bins + 1 > bins_cap) return fail(PKV_ERR_CAPACITY, "plan: %lld bins > bins_cap - 1", (long long)bins);
  const int64_t piece = std::max<int64_t>(1, total / (bins * pieces_per_bin));  // piece cap, in blocks
  const int64_t budget = (total * (100 - dyn_percent)) / (100 * bins);         // static load of a bin

  // pieces: sequence b in n_b even pieces of at most max(piece, ceil(blocks_b / max_splits)) blocks
  struct Piece {
    int32_t seq, first, end, slot;  // blocks [first, end) of sequence seq, split slot
  };
  std::vector<Piece> pieces;
  int32_t max_ns = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int64_t c = std::max(piece, ceil_div(blocks[b], max_splits));
    const int64_t n = ceil_div(blocks[b], c);
    for (int64_t j = 0; j < n; ++j)
      pieces.push_back({b, (int32_t)((j * blocks[b]) / n), (int32_t)(((j + 1) * blocks[b]) / n), (int32_t)j});
    n_splits_out[b] = (int32_t)n;
    max_ns = std::max(max_ns, (int32_t)n);
  }
  if ((int64_t)pieces.size() > work_cap)
    return fail(PKV_ERR_CAPACITY, "plan: %lld work items > work_cap=%d", (long long)pieces.size(), work_cap);
  // longest first; ties keep sequence, then piece order
  std::stable_sort(pieces.begin(), pieces.end(),
                   [](const Piece& x, const Piece& y) { return (x.end - x.first) > (y.end - y.first); });
  // every piece to the least loaded bin (lowest index among equals)
  std::vector<int64_t> load(bins, 0);
  std::vector<std::vector<int32_t>> in_bin(bins);
  for (int32_t i = 0; i < (int32_t)pieces.size(); ++i) {
    int64_t best = 0;
    for (int64_t k = 1; k < bins; ++k)
      if (load[k] < load[best]) best = k;
    load[best] += pieces[i].end - pieces[i].first;
    in_bin[best].push_back(i);
  }
  // bins give their last pieces (the smallest they got) to the queue while
  // over budget, keeping at least one; the queue runs longest first
  std::vector<int32_t> queue;
  for (int64_t k = 0; k < bins; ++k)
    while (in_bin[k].size() > 1 && load[k] > budget) {
      const int32_t i = in_bin[k].back();
      in_bin[k].pop_back();
      load[k] -= pieces[i].end - pieces[i].first;
      queue.push_back(i);
    }
  std::sort(queue.begin(), queue.end());  // sorted-piece index order = longest first, ties as above

  int64_t n = 0;
  auto emit = [&](int32_t i) {
    const Piece& pc = pieces[i];
    work_out[4 * n + 0] = pc.seq;
    work_out[4 * n + 1] = (int32_t)(kBalanceBlockKeys * pc.first);
    work_out[4 * n + 2] = (int32_t)(kBalanceBlockKeys * pc.end);
    work_out[4 * n + 3] = pc.slot;
    ++n;
  };
  bin_offsets_out[0] = 0;
  for (int64_t k = 0; k < bins; ++k) {
    for (int32_t i : in_bin[k]) emit(i);
    bin_offsets_out[k + 1] = (int32_t)n;
  }
  for (int32_t i : queue) emit(i);
  if (info) {
    info->num_work = (int32_t)n;
    info->num_real = (int32_t)n;
    info->chunk_tiles = (int32_t)ceil_div(piece, kTileKeys / kBalanceBlockKeys);
    info->slots = (int32_t)bins;
    info->max_n_splits = max_ns;
    info->num_bins = (int32_t)bins;
    info->num_dynamic = (int32_t)queue.size();
  }
  return PKV_OK;
}

// Plan choice. "MiniMax MSA fmha_sm100/cute README", Paged FP8 Decode: the
// schedule switches to load balancing when the kv-length distribution is
// imbalanced, max / avg >= 1.5. Reading: the lengths are those the one-wave
// plan hands to its workgroups (its work items, which already cut long
// sequences into chunks), in 32-key blocks of keys that exist.
// Paired plan (this library's own; see pkv_fp8.h): two work items per
// workgroup. The items of chunk c are those of the occupancy-pinned rule
// above; sorted longest first (ties in construction order) and padded with
// empty items to 2 * pair_slots entries, item k shares workgroup k with item
// 2 * pair_slots - 1 - k. The chunk is the smallest c >= ceil(T / max_splits)
// whose items fit (n <= 2 * pair_slots) and whose every pair holds at most c
// tiles, so that no workgroup carries more than a longest item alone.
extern "C" pkv_status pkv_plan_paired(const int32_t* seq_lens, int32_t num_seqs, int32_t pair_slots,
                                      int32_t max_splits, int32_t* work_out, int32_t work_cap,
                                      int32_t* n_splits_out, pkv_plan_info* info) {
  using pkv::fail;
  if (!seq_lens || !work_out || !n_splits_out) return fail(PKV_ERR_INVALID_ARG, "plan paired: NULL array");
  if (num_seqs < 1) return fail(PKV_ERR_INVALID_ARG, "plan paired: num_seqs=%d < 1", num_seqs);
  if (pair_slots < 1 || max_splits < 1 || work_cap < 0)
    return fail(PKV_ERR_INVALID_ARG, "plan paired: pair_slots=%d and max_splits=%d must be >= 1, work_cap=%d >= 0",
                pair_slots, max_splits, work_cap);
  if (max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_UNSUPPORTED, "plan paired: max_splits=%d > %d", max_splits, PKV_MAX_SPLITS);
  std::vector<int64_t> tiles(num_seqs);
  int64_t t_max = 1;
  for (int32_t b = 0; b < num_seqs; ++b) {
    if (seq_lens[b] < 0) return fail(PKV_ERR_INVALID_ARG, "plan paired: seq_lens[%d]=%d < 0", b, seq_lens[b]);
    tiles[b] = std::max<int64_t>(1, ceil_div(seq_lens[b], kTileKeys));
    t_max = std::max(t_max, tiles[b]);
  }
  const int64_t room = 2 * (int64_t)pair_slots;
  const int64_t lo = ceil_div(t_max, max_splits);
  std::vector<Item> items;
  auto build = [&](int64_t c) {
    items.clear();
    for (int32_t b = 0; b < num_seqs; ++b)
      for (int64_t j = 0; j * c < tiles[b]; ++j)
        items.push_back({b, (int32_t)(j * c), (int32_t)std::min((j + 1) * c, tiles[b]), (int32_t)j});
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& x, const Item& y) { return (x.end - x.begin) > (y.end - y.begin); });
  };
  auto len_at = [&](int64_t i) -> int64_t { return i < (int64_t)items.size() ? items[i].end - items[i].begin : 0; };
  int64_t chunk = -1;
  for (int64_t c = lo; c <= t_max && chunk < 0; ++c) {
    int64_t n = 0;
    for (int64_t t : tiles) n += ceil_div(t, c);
    if (n > room) continue;
    build(c);
    bool ok = true;
    for (int64_t k = 0; k < pair_slots && ok; ++k) ok = len_at(k) + len_at(room - 1 - k) <= c;
    if (ok) chunk = c;
  }
  if (chunk < 0)
    return fail(PKV_ERR_UNSUPPORTED, "plan paired: no chunk puts %d sequences into %d pairs of at most one chunk",
                num_seqs, pair_slots);
  const int64_t n = (int64_t)items.size();
  const int64_t pairs = std::min<int64_t>(pair_slots, n);
  if (2 * pairs > work_cap)
    return fail(PKV_ERR_CAPACITY, "plan paired: %lld work entries > work_cap=%d", (long long)(2 * pairs), work_cap);
  int32_t max_ns = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    n_splits_out[b] = (int32_t)ceil_div(tiles[b], chunk);
    max_ns = std::max(max_ns, n_splits_out[b]);
  }
  auto put = [&](int64_t e, int64_t i) {
    const Item it = i < n ? items[i] : Item{0, 0, 0, 0};
    work_out[4 * e + 0] = it.seq;
    work_out[4 * e + 1] = it.begin;
    work_out[4 * e + 2] = it.end;
    work_out[4 * e + 3] = it.slot;
  };
  for (int64_t k = 0; k < pairs; ++k) {
    put(2 * k, k);
    put(2 * k + 1, room - 1 - k);
  }
  if (info) {
    info->num_work = (int32_t)(2 * pairs);
    info->num_real = (int32_t)n;
    info->chunk_tiles = (int32_t)chunk;
    info->slots = (int32_t)std::min<int64_t>(room, INT32_MAX);
    info->max_n_splits = max_ns;
    info->num_bins = 0;
    info->num_dynamic = 0;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_plan_pick(const int32_t* seq_lens, int32_t num_seqs, const int32_t* work, int32_t num_work,
                                    int32_t kv_format, int32_t h_k, int32_t rows, int32_t* plan_out,
                                    float* imbalance_out) {
  using pkv::fail;
  if (!seq_lens || !work || !plan_out) return fail(PKV_ERR_INVALID_ARG, "plan pick: NULL argument");
  if (num_seqs < 1 || num_work < 0 || rows < 1 || h_k < 1) return fail(PKV_ERR_INVALID_ARG, "plan pick: bad sizes");
  int64_t total = 0, longest = 0, items = 0;
  for (int32_t i = 0; i < num_work; ++i) {
    const int32_t* w = work + 4 * i;
    if (w[0] < 0 || w[0] >= num_seqs || w[2] <= w[1]) continue;  // padding entries
    const int64_t L = std::max<int32_t>(seq_lens[w[0]], 0);
    const int64_t keys = std::min<int64_t>(w[2] * kTileKeys, L) - w[1] * kTileKeys;
    const int64_t blocks = std::max<int64_t>(1, ceil_div(std::max<int64_t>(keys, 0), kBalanceBlockKeys));
    total += blocks;
    longest = std::max(longest, blocks);
    ++items;
  }
  const float ratio = items ? (float)((double)longest * items / (double)total) : 1.0f;
  // the page's trigger, except where this library's balanced form measured
  // otherwise: the latent multi-token form (64 rows and more) restarts at an
  // item boundary at a cost of a few blocks, and gains from 1.12 on; the
  // narrow formats run the one-item form only
  const bool narrow = kv_format == PKV_KV_E2M1 || kv_format == PKV_KV_E2M3 || kv_format == PKV_KV_E3M2 ||
                      kv_format == PKV_KV_NVFP4;
  const float trigger = (kv_format == PKV_KV_MLA && rows >= 64) ? 1.12f : 1.5f;
  *plan_out = !narrow && ratio >= trigger ? PKV_PLAN_BALANCED : PKV_PLAN_WAVE;
  // four kv heads and one 16-row block: the paired plan, which the one-item
  // form runs at one eight-wave workgroup per CU (the streaming form behind
  // the balanced plan spends more per block than it gains). Measured on the
  // fully-fp8 batch, decode us one-wave -> paired: e4m3 169.3 -> 165.7, fp4
  // 103.9 -> 94.9, fp6 168 -> 152; NVFP4, whose one-wave plan already runs
  // two waves per SIMD, 146.9 -> 147.7 for the decode but 163.2 -> 161.1 for
  // decode + merge (16 splits instead of 32)
  if (kv_format != PKV_KV_MLA && h_k == 4 && rows <= 16) *plan_out = PKV_PLAN_PAIRED;
  if (imbalance_out) *imbalance_out = ratio;
  return PKV_OK;
}
