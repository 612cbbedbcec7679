/*
 * pkv_fp8.h -- C ABI of libpkvfp8.so: paged-KV e4m3 decode attention for
 * AMD MI355X (gfx950).
 *
 * What is computed. For every sequence b, KV head g and packed query row
 * n = qi * h_r + hr (h_r = h_q / h_k, qi-major: "mjolnir-kernel 0.1.0 wheel:
 * mjolnir/t5_decode.py", module docstring, "Query packing"), the row attends
 * to the keys j = 0 .. lim(n) of its sequence, lim(n) = L - q_len + qi under
 * the causal tail (q_len > 1, causal != 0) and L - 1 otherwise (block mode),
 * L = seq_lens[b] including the new tokens. Key j is row j % page_size of
 * page block_table[b][j / page_size]. With per-(sequence, kv-head) descales
 * qd, kd, vd ("Inputs follow vLLM's paged KV cache", same docstring):
 *   s_j = softmax_scale * qd * kd * <q, k_j>
 *   O[n] = o_scale * vd * sum_j exp(s_j - M) v_j / sum_j exp(s_j - M)
 *   LSE[n] = M + ln sum_j exp(s_j - M),   M = max_j s_j   (natural log)
 * A row that sees no key gets O = 0 and LSE = -inf (the page's epilogue and
 * reduction kernel). The latent-record variant (kv_format = PKV_KV_MLA;
 * "vLLM PR #62633", Kernel design) has one KV head whose key is 512 e4m3
 * latent values times one fp32 scale per 128-value block followed by 64 bf16
 * rope values, and whose value is the scaled latent part. The page
 * dequantises a record exactly to bf16, so the record's scales are read as
 * powers of two; the multi-token form (64 query rows and more) folds a
 * power-of-two scale into its bf16 key rows exactly and rounds the product
 * of any other scale to bf16, the other forms are exact for any scale.
 *
 * Call sequence (the page's module docstring, "Split-KV scheduling" and
 * "Workspace"; "MiniMax MSA fmha_sm100/cute README", Paged FP8 Decode,
 * plan() then run()):
 *   1. pkv_decode_slots()   -> CU count, resident workgroups per CU, q-row tiles
 *   2. pkv_plan_split_kv(), pkv_plan_even(), pkv_plan_balanced() or pkv_plan_queued() -> host
 *      work list + n_splits (+ bin offsets) (pure host code)
 *   3. copy work / n_splits to the device once (the caller's job)
 *   4. pkv_paged_decode_attn(); then pkv_merge_splits() when any sequence
 *      was split (info.max_n_splits > 1). Both only enqueue on `stream`:
 *      they never allocate, never synchronise and are capturable in a HIP
 *      graph; a plan made for upper-bound lengths stays valid for shorter
 *      runtime seq_lens.
 * The sparse slot-list decode needs no plan: pkv_sparse_decode() with a
 * workspace of pkv_sparse_workspace_bytes() (declared at the end).
 *
 * Ownership. The caller owns every buffer; the library keeps no state
 * between calls and never frees or retains a pointer. Device pointers are
 * plain device addresses (e.g. torch's data_ptr()).
 *
 * Errors. Every entry point returns a pkv_status. A call that fails
 * validation launches nothing and returns a negative code; nothing aborts or
 * throws across the ABI. pkv_last_error() gives a one-line reason for the
 * calling thread's most recent failure.
 *
 * Preconditions not checked on the device (a violation gives unspecified
 * results but no out-of-bounds access: page indices are clamped into
 * [0, num_pages) and L into [0, max_blocks * page_size], work items whose
 * sequence or split slot is out of range are skipped):
 *   block_table[b][i] in [0, num_pages) for i < ceil(L / page_size);
 *   descales positive and finite; the device work list and n_splits come
 *   from pkv_plan_split_kv with lengths >= the runtime seq_lens and the same
 *   max_splits.
 */
#ifndef PKV_FP8_H
#define PKV_FP8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1) /* null pointer, bad size, misaligned pointer or stride */
#define PKV_ERR_UNSUPPORTED (-2) /* valid request the library has no kernel for */
#define PKV_ERR_CAPACITY (-3)    /* an output array is too small (work_cap, pad_to) */
#define PKV_ERR_WORKSPACE (-4)   /* split workspace missing or too small */
#define PKV_ERR_HIP (-5)         /* the HIP runtime reported an error */

/* Static name of a status code ("PKV_OK", ...). Never NULL; an unknown code
 * gives "PKV_ERR_UNKNOWN".
 * The error convention follows the pages' rejections before any launch: the
 * kernel's can_implement ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py",
 * the decode class's can_implement: unsupported formats, head dim, head
 * ratio) maps to PKV_ERR_UNSUPPORTED / PKV_ERR_INVALID_ARG, and the plan()
 * step of "MiniMax MSA fmha_sm100/cute README" (Paged FP8 Decode, Known
 * Limitations: invalid lengths caught at plan time with a clear error) maps
 * to a negative status from the planner, with the reason in pkv_last_error().
 * Here the status is returned instead of raised, so no exception crosses the
 * C ABI. */
const char* pkv_status_string(pkv_status s);

/* Reason for the calling thread's most recent failing call (empty string if
 * none). The pointer stays valid until the thread's next failing call. */
const char* pkv_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

/* sizeof(pkv_decode_args) as compiled into the library, so that a binding
 * can check its own copy of the struct layout before the first call. */
size_t pkv_decode_args_size(void);

/* ------------------------------------------------------------------------ */
/* Split-KV planner (host only, pure: no GPU needed).                       */
/* ------------------------------------------------------------------------ */
typedef struct pkv_plan_info {
  int32_t num_work;     /* entries written to work_out (real + padding) */
  int32_t num_real;     /* non-empty work items */
  int32_t chunk_tiles;  /* 128-key tiles per chunk (a sequence's last chunk may be shorter) */
  int32_t slots;        /* work items that fit one wave of the grid */
  int32_t max_n_splits; /* largest n_splits over the batch */
  int32_t num_bins;     /* balanced / queued plan: workgroups (bins) of the grid; 0 for pkv_plan_split_kv */
  int32_t num_dynamic;  /* queued plan: items in the shared queue (after the bins' items); 0 otherwise */
} pkv_plan_info;

/*
 * Occupancy-pinned split-KV plan ("mjolnir-kernel 0.1.0 wheel:
 * mjolnir/t5_decode.py", plan_split_kv and the module docstring). In units
 * of 128-key tiles, tiles_b = max(1, ceil(L_b / 128)), T = max tiles_b:
 *   slots = max(1, cu_count * wg_per_cu / (h_k * n_q_tiles))
 *   lo    = max(min_chunk_tiles, ceil(T / max_splits))
 *   chunk = max(lo, ceil(T / force_splits))          if force_splits > 0
 *         = T                                         if num_seqs >= slots or max_splits == 1
 *         = smallest c >= lo with sum_b ceil(tiles_b / c) <= slots   otherwise
 * Sequence b becomes items (b, j*chunk, min((j+1)*chunk, tiles_b), j) for
 * j < n_splits[b] = ceil(tiles_b / chunk); items are ordered longest first
 * (ties keep sequence-major order); pad_to > 0 appends (0,0,0,0) items up to
 * pad_to entries, so a captured grid keeps one size.
 *
 * seq_lens      host int32[num_seqs], each >= 0
 * work_out      host int32[work_cap][4] (seq, tile_begin, tile_end, split_slot)
 * n_splits_out  host int32[num_seqs]
 * info          host, may be NULL
 * Errors: INVALID_ARG for num_seqs < 1, negative lengths, sizes < 1,
 * force_splits / pad_to < 0, NULL arrays; CAPACITY when the items do not fit
 * work_cap or exceed pad_to; UNSUPPORTED when a sequence would need more than
 * max_splits chunks (cannot happen for max_splits >= 1, kept as a guard) or
 * max_splits > PKV_MAX_SPLITS.
 */
#define PKV_MAX_SPLITS 256
pkv_status pkv_plan_split_kv(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                             int32_t cu_count, int32_t wg_per_cu, int32_t max_splits, int32_t force_splits,
                             int32_t min_chunk_tiles, int32_t pad_to, int32_t* work_out, int32_t work_cap,
                             int32_t* n_splits_out, pkv_plan_info* info);

/* Even plan (this library's own): the page's occupancy-pinned rule of
 * pkv_plan_split_kv at 32-key granularity. With blocks_b = max(1,
 * ceil(L_b / 32)), pick the smallest c >= ceil(max blocks / max_splits) with
 * sum_b ceil(blocks_b / c) <= slots (slots as in pkv_plan_split_kv; c = the
 * longest sequence's blocks when num_seqs >= slots), cut sequence b into
 * k_b = ceil(blocks_b / c) pieces, piece j covering blocks
 * [j * blocks_b / k_b, (j + 1) * blocks_b / k_b) (floors), and emit the items
 * (seq, key_begin, key_end, split_slot) in KEYS, longest first (stable).
 * Pieces of one sequence differ by at most one block, so the longest item is
 * shorter than with 128-key tiles. Run the decode with work_in_keys = 1.
 * info->chunk_tiles holds c in 32-key blocks. Errors as pkv_plan_split_kv. */
pkv_status pkv_plan_even(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles, int32_t cu_count,
                         int32_t wg_per_cu, int32_t max_splits, int32_t* work_out, int32_t work_cap,
                         int32_t* n_splits_out, pkv_plan_info* info);

/*
 * Balanced contiguous plan (this library's own planner; not from the pages).
 * The 32-key blocks of all sequences (max(1, ceil(L / 32)) each), laid end to
 * end in sequence order, are cut into `bins` contiguous shares of floor or
 * ceil(total / bins) blocks, bins = max(1, min(total, cu_count * wg_per_cu /
 * (h_k * n_q_tiles))) -- the workgroups that run at once -- lowered until no
 * sequence is cut into more than max_splits pieces. Every overlap of a share
 * and a sequence is a work item (seq, key_begin, key_end, split_slot) in KEYS
 * (not tiles): key_begin = 32 * its first block, key_end = min(32 * its end
 * block, L); split slots are numbered in key order. Items are listed bin by
 * bin and bin i owns items [bin_offsets[i], bin_offsets[i+1]). Each workgroup
 * then carries the same number of 32-key blocks (to one), whatever the length
 * mix; the decode streams a bin's items back to back through one load
 * pipeline.
 *
 * seq_lens        host int32[num_seqs], each >= 0
 * work_out        host int32[work_cap][4]; at most bins + num_seqs - 1 items
 * n_splits_out    host int32[num_seqs]
 * bin_offsets_out host int32[bins_cap], bins + 1 entries are written
 * info            host, may be NULL (num_bins = bins)
 * Errors: as pkv_plan_split_kv; CAPACITY when work_cap or bins_cap is too
 * small.
 */
pkv_status pkv_plan_balanced(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                             int32_t cu_count, int32_t wg_per_cu, int32_t max_splits, int32_t* work_out,
                             int32_t work_cap, int32_t* n_splits_out, int32_t* bin_offsets_out, int32_t bins_cap,
                             pkv_plan_info* info);

/*
 * Queued plan (this library's own planner; not from the pages). Its aim is
 * that the workgroups finish together, even when sequence lengths differ
 * and compute units or XCDs stream at different rates. With 32-key blocks
 * (max(1, ceil(L / 32)) per sequence), total = their sum and
 * bins = max(1, min(total, cu_count * wg_per_cu / (h_k * n_q_tiles))):
 *   piece  = max(1, floor(total / (bins * pieces_per_bin)))   piece cap, blocks
 *   budget = floor(total * (100 - dyn_percent) / (100 * bins)) static load of a bin
 *   c_b    = max(piece, ceil(blocks_b / max_splits))
 *   n_b    = ceil(blocks_b / c_b) pieces of sequence b; piece j covers blocks
 *            [floor(j * blocks_b / n_b), floor((j + 1) * blocks_b / n_b)) and
 *            uses split slot j (n_splits[b] = n_b).
 * Pieces are taken longest first (ties: sequence, then piece order). Each
 * goes to the bin with the smallest load (lowest index among equals). Bins
 * are then visited in order. While a bin holds more than one piece and its
 * load exceeds the budget, it moves its most recently assigned piece to the
 * queue. The queue runs in the same longest-first order. Work items are
 * (seq, key_begin, key_end, split_slot) in KEYS: key_begin = 32 * first
 * block, key_end = 32 * end block. key_end may pass L; the decode clamps to
 * the runtime length. Bin i's items are [bin_offsets[i], bin_offsets[i+1]).
 * The queue's items follow, [bin_offsets[bins], num_work).
 * The decode runs one persistent workgroup per bin, per kv-head group and
 * q-row tile. Each workgroup runs its bin's items, then takes queue items
 * until the queue is empty. Piece boundaries are fixed by the plan, so the
 * result does not depend on which workgroup ran which piece.
 *
 * seq_lens        host int32[num_seqs], each >= 0
 * pieces_per_bin  >= 1: pieces a bin's share is cut into (finer balance,
 *                 more split partials)
 * dyn_percent     share of the work kept for the queue, 0 .. 90
 * work_out        host int32[work_cap][4]
 * n_splits_out    host int32[num_seqs]
 * bin_offsets_out host int32[bins_cap]; bins + 1 entries are written
 * info            host, may be NULL (num_bins = bins, num_dynamic = queue length)
 * Errors: as pkv_plan_balanced; INVALID_ARG for pieces_per_bin < 1 or
 * dyn_percent outside [0, 90].
 */
pkv_status pkv_plan_queued(const int32_t* seq_lens, int32_t num_seqs, int32_t h_k, int32_t n_q_tiles,
                           int32_t cu_count, int32_t wg_per_cu, int32_t max_splits, int32_t pieces_per_bin,
                           int32_t dyn_percent, int32_t* work_out, int32_t work_cap, int32_t* n_splits_out,
                           int32_t* bin_offsets_out, int32_t bins_cap, pkv_plan_info* info);

/*
 * Plan choice ("MiniMax MSA fmha_sm100/cute README", Paged FP8 Decode: the
 * schedule balances the load when the kv-length distribution is imbalanced,
 * max / avg >= 1.5). The lengths compared are those of the one-wave plan's
 * work items (`work`, `num_work` as pkv_plan_split_kv wrote them, padding
 * entries skipped), in 32-key blocks of existing keys, max(1, ceil((min(end *
 * 128, L) - begin * 128) / 32)): imbalance = longest / mean. The plan is
 * PKV_PLAN_BALANCED (pkv_plan_balanced) when the imbalance reaches the
 * trigger of the decode form: 1.12 for the latent cache with rows >= 64 (its
 * multi-token form, measured on this part), 1.5 otherwise; always
 * PKV_PLAN_WAVE for the fp4, fp6 and NVFP4 caches (one-item form only).
 * With four kv heads and at most 16 rows (e4m3, fp4, fp6 and NVFP4 caches)
 * the balance comes from PKV_PLAN_PAIRED (pkv_plan_paired) instead, whatever
 * the imbalance: it runs the one-item form, and where the lengths are even it
 * pairs nothing and equals the one-wave plan (measured on this part, decode
 * one-wave -> paired on the fully-fp8 batch: e4m3 169.3 -> 165.7 us, fp4
 * 103.9 -> 94.9, fp6 168 -> 152; NVFP4 146.9 -> 147.7, but decode + merge
 * 163.2 -> 161.1, with half the splits).
 *
 * seq_lens   host int32[num_seqs]
 * work       host int32[num_work][4] (seq, tile_begin, tile_end, split_slot)
 * kv_format  PKV_KV_*; h_k kv heads; rows = q_len * h_q / h_k (packed query rows)
 * plan_out   PKV_PLAN_WAVE, PKV_PLAN_BALANCED or PKV_PLAN_PAIRED; imbalance_out
 *            may be NULL
 * Errors: INVALID_ARG for NULL pointers, num_seqs < 1, num_work < 0, rows < 1,
 * h_k < 1.
 */
#define PKV_PLAN_WAVE 0
#define PKV_PLAN_BALANCED 1
#define PKV_PLAN_PAIRED 2
pkv_status pkv_plan_pick(const int32_t* seq_lens, int32_t num_seqs, const int32_t* work, int32_t num_work,
                         int32_t kv_format, int32_t h_k, int32_t rows, int32_t* plan_out, float* imbalance_out);

/*
 * Paired plan (this library's own planner; not from the pages): the work
 * items of the occupancy-pinned rule (pkv_plan_split_kv) for a chunk of c
 * tiles, run two per workgroup. With tiles_b = max(1, ceil(L_b / 128)) and
 * T = max_b tiles_b, c is the smallest value >= ceil(T / max_splits) for
 * which the n = sum_b ceil(tiles_b / c) items fit 2 * pair_slots places and,
 * the items sorted longest first (ties in construction order: sequence,
 * then piece) and padded with empty items to 2 * pair_slots, item k and item
 * 2 * pair_slots - 1 - k together hold at most c tiles for every
 * k < pair_slots. Entries 2k and 2k+1 of work_out are the two items of
 * workgroup k, k < min(pair_slots, n); an empty item is (0, 0, 0, 0).
 * Run the decode with work_pairs = 1. pair_slots: the workgroups of two
 * items that run at once (one per CU for four kv heads: 8 waves).
 *
 * Why: with one item per workgroup, sequences shorter than the chunk leave
 * CUs idle while the longest chunks stream at one CU's rate; pairing the
 * shortest items frees places for a smaller chunk (measured on the
 * fully-fp8 workload: 171 -> 166-167 us).
 *
 * seq_lens      host int32[num_seqs], >= 0
 * work_out      host int32[work_cap][4] (seq, tile_begin, tile_end, split_slot)
 * n_splits_out  host int32[num_seqs]
 * Errors: INVALID_ARG for NULL arrays, num_seqs < 1, pair_slots < 1,
 * max_splits < 1, negative lengths; UNSUPPORTED for max_splits > PKV_MAX_SPLITS
 * or when no chunk satisfies the rule (more sequences than the pairs can
 * hold at one chunk each); CAPACITY when 2 * min(pair_slots, n) > work_cap.
 * info (optional): num_work = 2 * min(pair_slots, n), num_real = n,
 * chunk_tiles = c, slots = 2 * pair_slots, max_n_splits, num_bins = 0.
 */
pkv_status pkv_plan_paired(const int32_t* seq_lens, int32_t num_seqs, int32_t pair_slots, int32_t max_splits,
                           int32_t* work_out, int32_t work_cap, int32_t* n_splits_out, pkv_plan_info* info);

/* ------------------------------------------------------------------------ */
/* Decode launch arguments                                                   */
/* ------------------------------------------------------------------------ */
#define PKV_Q_BF16 0 /* q is bf16; q_descale is ignored */
#define PKV_Q_E4M3 1 /* q is e4m3 codes with q_descale */

#define PKV_KV_E4M3 0 /* K and V caches of e4m3 codes, d_qk = d_v = 128 */
#define PKV_KV_MLA 1  /* latent records: h_k = 1, d_qk = 576 (512 latent + 64 rope), d_v = 512 */
/* Packed fp4 K and V caches ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py",
 * narrow KV formats): e2m1 codes (1 sign, 2 exponent bits with bias 1, 1
 * mantissa bit; no inf/NaN), a row of d = 128 codes in 64 bytes with element
 * 2i in the low nibble of byte i; the usual per-(sequence, kv-head) descales;
 * d_qk = d_v = 128 and an e4m3 query (PKV_Q_E4M3); one-wave plan only (no
 * bin_offsets / queue). */
#define PKV_KV_E2M1 2
/* Packed fp6 K and V caches (the same page's KV cache formats "e2m3" and
 * "e3m2", and pack_subbyte): e2m3 codes (1 sign, 2 exponent bits with bias 1,
 * 3 mantissa bits; largest 7.5) or e3m2 codes (1 sign, 3 exponent bits with
 * bias 3, 2 mantissa bits; largest 28), no inf/NaN; a row of d = 128 codes in
 * 96 bytes read as one little-endian bitstream, element i at bits 6i..6i+5;
 * per-(sequence, kv-head) descales; d_qk = d_v = 128, an e4m3 query and the
 * one-wave plan only, as for PKV_KV_E2M1. */
#define PKV_KV_E2M3 3
#define PKV_KV_E3M2 4
/* NVFP4 K and V caches (the same page's "nvfp4" and nvfp4_quantize): rows
 * packed as for PKV_KV_E2M1 plus one e4m3 scale per 16 head-dim values in
 * k_group_scale / v_group_scale. The decode multiplies the values
 * e4m3(code * scale * 2^-3) (rounded to nearest, ties to even; the product
 * is at most 336, so nothing saturates) times the per-(sequence, kv-head)
 * descales, which carry the 2^3 back. d_qk = d_v = 128, an e4m3 query and
 * the one-wave plan only. */
#define PKV_KV_NVFP4 5

/*
 * All strides are in ELEMENTS of the pointed-to type, >= 0; a descale
 * stride of 0 broadcasts (per-tensor, per-head or per-(seq, head) scales).
 * Tensor layouts ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", module
 * docstring and kernel_strides; logical views of any physical layout with
 * the last dimension contiguous):
 *   q      [num_seqs * q_len][h_q][d_qk]     bf16 or e4m3  (q_tok_stride, q_head_stride)
 *   k, v   [num_pages][page_size][h_k][d]    e4m3 codes    (page, row, head strides, bytes)
 *          PKV_KV_E2M1: [num_pages][page_size][h_k][d/2] packed fp4 bytes (byte strides)
 *          PKV_KV_E2M3 / E3M2: [num_pages][page_size][h_k][3d/4] packed fp6 bytes (byte strides)
 *          PKV_KV_NVFP4: as PKV_KV_E2M1, plus the group scales (k/v_group_scale)
 *          MLA: k = v = latent [pages][PS][1][512] e4m3 (v may be NULL or equal k)
 *   k_rope MLA only: [pages][PS][1][64] bf16 (page, row strides)
 *   k_blk_scale MLA only: [pages][PS][1][4] fp32, one scale per 128 latent values
 *          (a power of two in the record format; pkv_write_kv writes such scales)
 *   block_table [num_seqs][max_blocks] int32 (bt_row_stride)
 *   seq_lens    [num_seqs] int32
 *   q/k/v_descale fp32 at [b * seq_stride + g * head_stride] (unused for MLA)
 *   o      [num_seqs * q_len][h_q][d_v] bf16 (o_tok_stride, o_head_stride)
 *   lse    [num_seqs][h_k][q_len * h_r] fp32, contiguous
 *   work   [num_work][4] int32 from pkv_plan_split_kv (device copy)
 *   n_splits [num_seqs] int32 from pkv_plan_split_kv (device copy)
 *   workspace  >= pkv_workspace_bytes(...) bytes of device memory, 256-B
 *          aligned, NOT initialised (only the splits a sequence used are
 *          read back); may be NULL when max_splits == 1.
 * Alignment: q, k, v, o and workspace 16-byte aligned, and every stride of
 * q, k, v and o a multiple of 16 bytes (8-byte multiples for e4m3 q).
 * Limits (UNSUPPORTED beyond them): page_size * row stride below 2^30 bytes
 * (in-page offsets are 32-bit) and every page stride of k, v and the NVFP4
 * group scales below 2^32 bytes (page offsets are 32 x 32-bit products).
 */
typedef struct pkv_decode_args {
  int32_t num_seqs, q_len, h_q, h_k, d_qk, d_v;
  int32_t page_size, num_pages, max_blocks;
  int32_t causal;    /* nonzero: causal tail for q_len > 1; zero: block mode */
  int32_t q_format;  /* PKV_Q_* */
  int32_t kv_format; /* PKV_KV_* */
  float softmax_scale;
  float o_scale; /* output multiplier (1.0 for plain attention) */

  const void* q;
  int64_t q_tok_stride, q_head_stride;
  const uint8_t* k;
  int64_t k_page_stride, k_row_stride, k_head_stride;
  const uint8_t* v;
  int64_t v_page_stride, v_row_stride, v_head_stride;
  const uint16_t* k_rope;
  int64_t rope_page_stride, rope_row_stride;
  const float* k_blk_scale;
  int64_t scale_page_stride, scale_row_stride;

  const int32_t* block_table;
  int64_t bt_row_stride;
  const int32_t* seq_lens;

  const float* q_descale;
  int64_t qd_seq_stride, qd_head_stride;
  const float* k_descale;
  int64_t kd_seq_stride, kd_head_stride;
  const float* v_descale;
  int64_t vd_seq_stride, vd_head_stride;

  void* o;
  int64_t o_tok_stride, o_head_stride;
  float* lse;

  const int32_t* work;
  int32_t num_work;
  const int32_t* n_splits;
  int32_t max_splits;
  void* workspace;
  size_t workspace_bytes;
  /* Optional, device int32[num_bins + 1] from pkv_plan_balanced: workgroup i
   * streams work items [bin_offsets[i], bin_offsets[i+1]) in order, the grid
   * has num_bins workgroups per (kv-head group, q-row tile), and `work` holds
   * KEY ranges (key_begin a multiple of 32), as pkv_plan_balanced writes
   * them. NULL: one work item per workgroup, num_work workgroups, and `work`
   * holds 128-key TILE ranges (pkv_plan_split_kv). */
  const int32_t* bin_offsets;
  int32_t num_bins;
  /* Optional, device int32[2 * h_k * n_q_tiles] (e4m3 K/V cache only), for a
   * plan from pkv_plan_queued: when non-NULL (bin_offsets required), the
   * grid has num_bins persistent workgroups per (kv-head group, q-row tile).
   * Each runs the items of its bin one after another, then takes queue
   * items [bin_offsets[num_bins], num_work) from a shared counter until none
   * is left. The counters must be zero before the first call. Every
   * completed call leaves them zero (the last workgroup to finish resets
   * them), so no per-call clearing is needed and the launch can be replayed
   * in a HIP graph. Calls that overlap on one counter array race. */
  int32_t* queue;
  /* PKV_KV_NVFP4 only (NULL otherwise): the e4m3 group scales of K and V,
   * one byte per 16 head-dim values, [num_pages][page_size][h_k][d/16] with
   * byte strides; k_group_scale 8-B aligned with 8-B multiple strides. */
  const uint8_t* k_group_scale;
  int64_t kgs_page_stride, kgs_row_stride, kgs_head_stride;
  const uint8_t* v_group_scale;
  int64_t vgs_page_stride, vgs_row_stride, vgs_head_stride;
  /* 1: the work items' ranges are in keys (pkv_plan_even; every key_begin a
   * multiple of 32, else the item is skipped), 0: in 128-key tiles
   * (pkv_plan_split_kv). The balanced and queued plans are in keys whatever
   * this says. e4m3 and narrow caches only. */
  int32_t work_in_keys;
  /* 1: `work` holds pairs (pkv_plan_paired): workgroup k runs entries 2k and
   * 2k+1 with one wave per (entry, kv head), num_work even. Needs h_k = 4,
   * q_len * h_q / h_k <= 16, an e4m3 or narrow cache, no bin_offsets and
   * work_in_keys = 0. 0: one entry per workgroup. */
  int32_t work_pairs;
} pkv_decode_args;

/* Bytes of split workspace: max_splits * num_seqs * h_k * n_rows * (d_v + 2)
 * fp32 values (partial O, max and sum per row and split), rounded up to 256.
 * ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", module docstring,
 * "Workspace": the o/m/l partials need no initialisation, because the merge
 * reads only the split slots a sequence used and padding items exit at once.)
 * The caller allocates it (device memory, 256-B aligned) and keeps it for as
 * long as the plan is used; its contents between calls do not matter.
 * Returns 0 when an argument is < 1 (no workspace can be sized). */
size_t pkv_workspace_bytes(int32_t num_seqs, int32_t h_k, int32_t n_rows, int32_t d_v, int32_t max_splits);

/*
 * Occupancy facts the planner needs for these arguments (shapes, formats,
 * mode; pointers are not read): the current device's compute-unit count,
 * how many (work item, kv head, q-row tile) units to plan per CU, and the
 * number of q-row tiles of the grid. For the e4m3 cache a unit is one wave
 * and the count targets about four streaming waves per CU (at least one
 * workgroup, at most what fits); for the latent cache a unit is one
 * workgroup and the count is the resident maximum. Queries the HIP runtime; no
 * launch. Errors: INVALID_ARG / UNSUPPORTED as pkv_paged_decode_attn would
 * return for the shapes, HIP on a runtime failure.
 */
pkv_status pkv_decode_slots(const pkv_decode_args* a, int32_t* cu_count, int32_t* wg_per_cu,
                            int32_t* n_q_tiles);

/*
 * Name of the device kernel that pkv_paged_decode_attn launches for these
 * arguments ("gqa_decode_kernel", "mla_pair_kernel" or "mla_lds_kernel"), so
 * that profiler output can be matched to a call. Host only, launches nothing.
 * Returns a static string, or NULL when the shapes fail validation
 * (pkv_last_error() says why).
 */
const char* pkv_decode_kernel_name(const pkv_decode_args* a);

/*
 * Split-KV decode ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py",
 * decode kernel: online softmax over the work item's contiguous key range,
 * then its epilogue). One workgroup per (work item, kv head, q-row tile).
 * A sequence with n_splits == 1 writes its final bf16 O and LSE directly; a
 * split one writes fp32 partials (O * vd, max in natural-log units, sum) to
 * its split slot of the workspace. Empty (padding) items exit at once.
 * `stream` is a hipStream_t (NULL = the null stream). Validates everything
 * before launching; returns HIP if the launch itself fails.
 */
pkv_status pkv_paged_decode_attn(const pkv_decode_args* a, void* stream);

/*
 * Combine of split partials ("mjolnir-kernel 0.1.0 wheel:
 * mjolnir/t5_decode.py", reduction kernel): for every sequence with
 * n_splits > 1 and every row, m* = max_j m_j, w_j = exp(m_j - m*) (0 for
 * m_j = -inf), O = o_scale * sum_j w_j O_j / sum_j w_j l_j (0 if the sum is
 * 0), LSE = m* + ln sum_j w_j l_j, over j < n_splits[b] in index order.
 * Sequences with n_splits <= 1 are left as the decode wrote them. A no-op
 * (nothing launched) when max_splits == 1. Same arguments as the decode.
 */
pkv_status pkv_merge_splits(const pkv_decode_args* a, void* stream);

/* ---- producers either side of the decode ---------------------------------- */

/*
 * Query quantisation for the fully-fp8 path ("mjolnir-kernel 0.1.0 wheel:
 * mjolnir/t5_decode.py", quantize_q_fp8). Per sequence b and kv head g:
 *   amax = max(|q|) over the sequence's q_len tokens, the h_r = h_q / h_k
 *          query heads g*h_r .. g*h_r + h_r - 1 and the d values (at least 1e-6)
 *   q_descale[b][g] = amax / 448                                  (fp32)
 *   q8 = e4m3 code of q / q_descale[b][g], round to nearest even  (fp32 division)
 * so the largest |q| of each group maps to +-448. One launch, no workspace,
 * no synchronisation (capturable).
 *
 * q          device bf16 [num_seqs * q_len][h_q][d]; strides in elements, d
 *            contiguous; 16-B aligned, strides multiples of 8 elements
 * q8         device uint8 (e4m3) of the same logical shape; strides in bytes,
 *            multiples of 8, 8-B aligned; may not overlap q
 * q_descale  device fp32 [num_seqs][h_k] with element strides (>= 0)
 * Errors: INVALID_ARG for sizes < 1, h_q % h_k != 0, d not a multiple of 8,
 * NULL or misaligned pointers, bad strides; HIP if the launch fails.
 */
typedef struct pkv_quant_q_args {
  int32_t num_seqs, q_len, h_q, h_k, d;
  const void* q;
  int64_t q_tok_stride, q_head_stride;
  uint8_t* q8;
  int64_t q8_tok_stride, q8_head_stride;
  float* q_descale;
  int64_t qd_seq_stride, qd_head_stride;
} pkv_quant_q_args;

pkv_status pkv_quantize_q(const pkv_quant_q_args* a, void* stream);

/* sizeof(pkv_quant_q_args) as compiled (a binding's layout check) */
size_t pkv_quant_q_args_size(void);

/*
 * Paged KV-cache write of the newest tokens (the "KV-cache write" that the
 * t5_decode page names among the kernels before the decode, with the
 * per-(sequence, kv head) e4m3 storage of its module docstring and harness;
 * the latent record of "vLLM PR #62633", Kernel design). Token t (0 <= t <
 * n_new) of sequence b is position pos = seq_lens[b] - n_new + t (seq_lens
 * already count the new tokens); it is written to row pos % page_size of page
 * block_table[b][pos / page_size]. Tokens with pos < 0, or whose block-table
 * entry lies outside [0, num_pages), are skipped.
 *   PKV_KV_E4M3: k[page][row][g][:] = e4m3(k_new[b*n_new + t][g][:] / k_descale[b][g]),
 *                likewise v; round to nearest even, |x| beyond 448 saturates to
 *                +-448, NaN gives 0x7F.
 *   PKV_KV_MLA:  h_k = 1 and d = 576; per token and 128-value latent block j:
 *                scale_j = the smallest power of two >= max(amax_j, 1e-6) / 448 (fp32),
 *                k_blk_scale[page][row][j] = scale_j,
 *                k[page][row][128j + i] = e4m3(x[128j + i] / scale_j); the 64
 *                rope values are copied bit for bit into k_rope. v_* unused.
 * One launch, no workspace, no synchronisation (capturable). Tokens written
 * by one call must map to distinct cache rows.
 *
 * k_new, v_new   device bf16 [num_seqs * n_new][h_k][d] (latent: [..][576],
 *                head stride unused); element strides; 16-B aligned, strides
 *                multiples of 8 elements, d contiguous
 * k, v           device uint8 caches with byte strides (page, row, head),
 *                8-B aligned, strides multiples of 8
 * k_rope, k_blk_scale  (latent) element strides (page, row), 16-B aligned
 * Errors: INVALID_ARG for sizes < 1, NULL or misaligned pointers, bad
 * strides, d not a multiple of 8 (e4m3) or not 576 (latent); UNSUPPORTED for
 * a page size outside {16, 32, 64, 128}; HIP if the launch fails.
 */
typedef struct pkv_kv_write_args {
  int32_t num_seqs, n_new, h_k, d, page_size, num_pages, max_blocks;
  int32_t kv_format; /* PKV_KV_* */
  const void* k_new;
  int64_t kn_tok_stride, kn_head_stride;
  const void* v_new;
  int64_t vn_tok_stride, vn_head_stride;
  const int32_t* block_table;
  int64_t bt_row_stride;
  const int32_t* seq_lens;
  const float* k_descale;
  int64_t kd_seq_stride, kd_head_stride;
  const float* v_descale;
  int64_t vd_seq_stride, vd_head_stride;
  uint8_t* k;
  int64_t k_page_stride, k_row_stride, k_head_stride;
  uint8_t* v;
  int64_t v_page_stride, v_row_stride, v_head_stride;
  uint16_t* k_rope;
  int64_t rope_page_stride, rope_row_stride;
  float* k_blk_scale;
  int64_t scale_page_stride, scale_row_stride;
} pkv_kv_write_args;

pkv_status pkv_write_kv(const pkv_kv_write_args* a, void* stream);

/* sizeof(pkv_kv_write_args) as compiled (a binding's layout check) */
size_t pkv_kv_write_args_size(void);

/* ------------------------------------------------------------------------ */
/* Sparse slot-list decode over latent records                               */
/* ------------------------------------------------------------------------ */
/*
 * "vLLM PR #62633: swap-AB CuTe DSL decode attention for DeepSeek-V4.1",
 * Kernel design: each decode token attends to the records named by its slot
 * lists (a sliding-window list and a top-k list of compressed records), the
 * record serving as key and value (S = KV Q^T, O = KV^T P, P split into bf16
 * hi and lo parts), and the token's tile partials are merged together with
 * a per-head attention sink. The record is the latent record of PKV_KV_MLA
 * (512 e4m3 codes, one fp32 scale per 128 codes, 64 bf16 rope values); the
 * model's own record format is not built.
 *
 * For token t and head h, over the non-negative entries s of both lists
 * (a slot is row s % page_size of page s / page_size of that list's pool;
 * an entry listed twice counts twice):
 *   z_s = softmax_scale * <q[t][h], key_s>
 *   Z   = sum_s exp(z_s) + exp(sink[h])            (no sink term if sink == NULL)
 *   o[t][h]   = o_scale * sum_s exp(z_s) value_s / Z   (bf16)
 *   lse[t][h] = log Z   (natural log; O = 0 and LSE = -inf when Z = 0)
 */
typedef struct pkv_sparse_list {
  const uint8_t* latent;    /* [num_pages][page_size] records: 512 e4m3 codes (bytes) */
  int64_t lat_page_stride, lat_row_stride;        /* bytes */
  const uint16_t* rope;     /* [num_pages][page_size][64] bf16 */
  int64_t rope_page_stride, rope_row_stride;      /* bf16 elements */
  const float* blk_scale;   /* [num_pages][page_size][4] fp32 */
  int64_t scale_page_stride, scale_row_stride;    /* fp32 elements */
  int32_t page_size;        /* 16, 32, 64 or 128 */
  int32_t num_pages;
  const int32_t* slots;     /* device [num_tokens][width] int32, row stride slots_row_stride; < 0: none */
  int64_t slots_row_stride;
  int32_t width;            /* entries per token, 0 .. 4096; 0 = list unused (pointers may be NULL) */
} pkv_sparse_list;

typedef struct pkv_sparse_args {
  int32_t num_tokens;       /* decode tokens, 1 .. 65535 */
  int32_t h_q;              /* query heads, a multiple of 16, <= 128 */
  const uint16_t* q;        /* [num_tokens][h_q][576] bf16 (q_tok_stride, q_head_stride in elements) */
  int64_t q_tok_stride, q_head_stride;
  /* list 0: sliding window; list 1: top-k compressed records; each list is
   * processed in tiles of 64 slots (the page cuts the top-k list into 128) */
  pkv_sparse_list list[2];
  const float* sink;        /* device [h_q] fp32 logits in scaled-score units, or NULL */
  float softmax_scale, o_scale;
  uint16_t* o;              /* [num_tokens][h_q][512] bf16 (o_tok_stride, o_head_stride in elements) */
  int64_t o_tok_stride, o_head_stride;
  float* lse;               /* device [num_tokens][h_q] fp32, contiguous */
  void* workspace;          /* >= pkv_sparse_workspace_bytes(a) bytes, 256-B aligned, never initialised */
  int64_t workspace_bytes;
} pkv_sparse_args;

/* Bytes of tile partials one call needs: tiles * num_tokens * h_q * (512 + 2)
 * fp32, tiles = ceil(width0 / 64) + ceil(width1 / 64); 0 on invalid args. */
int64_t pkv_sparse_workspace_bytes(const pkv_sparse_args* a);

/* Two launches on `stream` (a hipStream_t; NULL = default stream): the tile
 * kernel (one workgroup per (token, tile, 16 or 32 heads), tile partials to
 * the workspace) and the merge (partials in tile order, list 0 first, plus
 * the sink). Allocates nothing, does not synchronise. Errors before any
 * launch: PKV_ERR_INVALID_ARG (NULL or misaligned pointers, bad strides or
 * sizes), PKV_ERR_UNSUPPORTED (page size, h_q, width limits),
 * PKV_ERR_WORKSPACE (missing or short workspace), PKV_ERR_HIP (a launch
 * failed). Slots past a pool are treated as absent (never read). */
pkv_status pkv_sparse_decode(const pkv_sparse_args* a, void* stream);

/* The two launches of pkv_sparse_decode separately (same checks, same
 * errors): the tile kernel, which writes the tile partials to the workspace,
 * and the merge, which reads them; pkv_sparse_merge must follow a
 * pkv_sparse_tiles call with the same arguments on the same stream. */
pkv_status pkv_sparse_tiles(const pkv_sparse_args* a, void* stream);
pkv_status pkv_sparse_merge(const pkv_sparse_args* a, void* stream);

/* sizeof(pkv_sparse_args) as compiled (a binding's layout check) */
size_t pkv_sparse_args_size(void);

/* ------------------------------------------------------------------------ */
/* Decode step that allocates nothing.                                      */
/* ------------------------------------------------------------------------ */
/* Bytes of split workspace the library holds per device for
 * pkv_paged_decode_noalloc (64 MiB). */
#define PKV_NOALLOC_WORKSPACE_BYTES (64u << 20)

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode step as pkv_paged_decode_attn followed by pkv_merge_splits, with the
 * split workspace taken from a device array the library holds (one per
 * device, PKV_NOALLOC_WORKSPACE_BYTES, kept from the first call on that
 * device until the process ends) instead of a->workspace, which is ignored.
 * The caller still passes every input and output, the work list and
 * n_splits. The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); its first call on a device looks the array's address up.
 *
 * Every call on a device shares that device's array and finds the previous
 * call's contents there; the workspace needs no initialisation (the merge
 * reads only the split slots this call's decode wrote), but calls that
 * overlap in time on one device (other streams, other threads) race on it
 * and give undefined results. Serialise them.
 *
 * Errors, before any launch: those of pkv_paged_decode_attn;
 * PKV_ERR_WORKSPACE when pkv_workspace_bytes(num_seqs, h_k, q_len * h_q / h_k,
 * d_v, max_splits) exceeds PKV_NOALLOC_WORKSPACE_BYTES (max_splits == 1 needs
 * none); PKV_ERR_UNSUPPORTED with queue set (the queued plan keeps counters
 * of its own).
 */
pkv_status pkv_paged_decode_noalloc(const pkv_decode_args* a, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement: streaming-read probe.                                       */
/* ------------------------------------------------------------------------ */
/*
 * Reads `bytes` of device memory at `src` once with plain coalesced 16-byte
 * loads and does nothing else, so that the HBM read rate of the decode
 * kernels can be stated as a fraction of what this part reaches for a pure
 * read in the same session ("mjolnir-kernel 0.1.0 wheel:
 * mjolnir/t5_decode.py", `run`: GB/s = bytes moved / kernel time; this is
 * that figure for a kernel that only streams).
 *
 * One launch of `workgroups` workgroups of 256 threads; each lane issues
 * `unroll` (4, 8 or 16) independent 16-byte loads per step, and the
 * workgroups walk 4 KiB * unroll chunks grid-stride. Nothing the kernel
 * reads reaches an output; `sink` (device, >= workgroups uint32 values) is
 * written only in the case that a lane's XOR of its words equals a fixed
 * pattern, which keeps the loads from being optimised away.
 *
 * src   device, 16-B aligned; bytes > 0 and a multiple of 4096 * unroll.
 * Errors before any launch: PKV_ERR_INVALID_ARG (NULL or misaligned
 * pointers, sizes out of range); PKV_ERR_HIP (the launch failed). Allocates
 * nothing, does not synchronise.
 */
pkv_status pkv_stream_read_probe(const void* src, size_t bytes, int32_t workgroups, int32_t unroll, uint32_t* sink,
                                 void* stream);

/*
 * Per-phase timestamps of a decode main loop (measurement only; no passage of
 * the sources: it shows where the time of a loop step goes). A library built
 * with -DPKV_STAMPS=1 records, in lane 0 of each wave (at most 8) of
 * workgroups 0..15 whose blockIdx.y and .z are 0, the shader clock
 * (s_memtime) at up to 8 points of each of the first 48 steps of the
 * workgroup's first work item:
 *   loop 0, the one-item form of the kv-head decode, per 32-key block:
 *     0 block start, 1 its fetch issued, 2 its loads landed, 3 processed;
 *   loop 1, the latent kernels (one buffer for both forms):
 *     the staged form, per 32-key step (from the second): 0 step start,
 *     1 loads issued and converted, 2 MFMA phase done, 3 past the first
 *     barrier, 4 softmax done, 5 past the second barrier;
 *     the pair form, per 16-key block: 0 block start, 1 its fetch issued,
 *     2 its loads landed, 3 partial S stored, 4 past the exchange barrier,
 *     5 softmax done, 6 PV issued.
 * Stamps of the last launch of that loop are copied (synchronously) to
 * host_dst, PKV_STAMP_WORDS uint64 values laid out as
 * [workgroup 16][wave 8][step 48][point 8]; entries never written stay as
 * the previous launches left them (zero at load).
 * Errors: PKV_ERR_INVALID_ARG (NULL host_dst, loop not 0 or 1),
 * PKV_ERR_UNSUPPORTED (a library built without the stamps: the normal
 * build), PKV_ERR_HIP (the copy failed).
 */
#define PKV_STAMP_WORDS (16 * 8 * 48 * 8)
pkv_status pkv_debug_stamps(int32_t loop, uint64_t* host_dst);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* PKV_FP8_H */
