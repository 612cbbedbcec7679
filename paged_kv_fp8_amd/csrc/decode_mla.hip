// Split-KV paged decode over latent records (MLA-like), gfx950.
//
// Method: the decode of "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py"
// (module docstring: work items, causal tail, direct write / partials; the
// decode kernel's online softmax) applied to the record cache of "vLLM PR
// #62633" (Kernel design): one KV head whose key j is its 512 e4m3 latent
// values times one fp32 scale per 128-value block, followed by 64 bf16 rope
// values, and whose value is the scaled latent part. Row n = qi * h_q + h
// (qi-major) sees keys 0 .. lim(n) as in the GQA path.
//
// gfx950 design (two forms, by query rows per sequence):
//  * The per-128 block scales are not multiplied into the e4m3 codes (the
//    product is not a bf16 value in general): QK^T keeps one fp32
//    accumulator per 128-value block and combines them with each key's
//    scales, s = sum_blk scale_blk * <q_blk, code_blk> + <q_rope, rope>; PV
//    multiplies P by the key's block scale (one bf16 P operand per 128-value
//    block of d_v), so V stays the exact codes. The codes convert to bf16
//    exactly (v_cvt_scalef32_pk_bf16_fp8 with scale 1).
//  * QK^T on v_mfma_f32_16x16x32_bf16 with keys on M; the V^T operand comes
//    from bf16 key rows in LDS through the transpose load, so P stays in the
//    lanes that computed it.
//  * Fewer than 64 rows (one to three query tokens): the pair form, two waves
//    per 16 rows that split each record by d_v half and exchange partial S.
//  * 64 rows and more: the staged form, four waves (one per SIMD) that share
//    one bf16 copy of each 32-key block in LDS, with the record's
//    power-of-two block scales folded into it.
//  * Load discipline as in the GQA kernel: every fetch issues the same loads
//    (keys clamped to the chunk's last key), the page of a block comes from a
//    one-dword vector load issued early enough that its wait covers only the
//    block being consumed, the loop runs whole rounds.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pkv_internal.h"
#include "stamps.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDv = 512;
constexpr int kTileKeys = 128;  // planner tile
constexpr int kBlockKeys = 16;  // keys per pair-form step
constexpr float kLazyLog2 = 8.0f;  // bf16 P: reference max may lag until p would exceed 2^8

struct MlaParams {
  const uint8_t* q;
  int64_t q_tok, q_head;  // bytes
  const uint8_t* lat;
  int64_t lat_page, lat_row;  // bytes
  const uint8_t* rope;
  int64_t rope_page, rope_row;  // bytes
  const uint8_t* scl;
  int64_t scl_page, scl_row;  // bytes
  const int32_t* block_table;
  int64_t bt_row;
  const int32_t* seq_lens;
  uint8_t* o;
  int64_t o_tok, o_head;  // bytes
  float* lse;
  const int4* work;
  const int32_t* n_splits;
  float* ws_o;    // [max_splits][num_seqs][rows][512]
  float2* ws_ml;  // [max_splits][num_seqs][rows]
  const int32_t* bin_offsets;  // [bins + 1] or null: one work item per workgroup
  float scale_log2e, scale, o_scale;
  int num_seqs, q_len, h_q, rows, page_shift, num_pages, max_blocks, max_splits;
};

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint2 x) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// codes x record block scale, as bf16. The scaled convert applies only the
// exponent of its scale operand, so it is exact, and the product, when the
// scale is a normal power of two (the record format's scales); any other
// scale takes the fp32 product, rounded to bf16.
__device__ __forceinline__ bf16x8 e4m3x8_times_pow2(uint2 x, float s) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, s, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, s, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, s, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, s, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ bf16x8 e4m3x8_times_any(uint2 x, float s) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(x.x, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.x, true),
                        __builtin_amdgcn_cvt_pk_f32_fp8(x.y, false), __builtin_amdgcn_cvt_pk_f32_fp8(x.y, true)};
  bf16x8 r;
  for (int h = 0; h < 4; ++h) {
    const bf16x2 o = __builtin_convertvector((f32x2_t){v[h][0] * s, v[h][1] * s}, bf16x2);
    r[2 * h] = o[0];
    r[2 * h + 1] = o[1];
  }
  return r;
}
// true when every one of the four fp32 scales is a normal power of two
__device__ __forceinline__ bool pow2_scales(uint4 s) {
  const uint32_t lo = min(min(s.x, s.y), min(s.z, s.w)), hi = max(max(s.x, s.y), max(s.z, s.w));
  return ((s.x | s.y | s.z | s.w) & 0x807FFFFFu) == 0 && lo >= 0x00800000u && hi <= 0x7F000000u;
}

__device__ __forceinline__ uint2 half_of(uint4 x, int h) { return h ? uint2{x.z, x.w} : uint2{x.x, x.y}; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) {
  bf16x8 r;
  __builtin_memcpy(&r, &x, 16);
  return r;
}

// max of two and of three, written out: through fmaxf the compiler first
// canonicalises each operand that comes from an MFMA or a lane swap (a v_max
// of the value with itself), which doubles the work. No operand here is a
// signalling NaN.
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// two fp32 values as one packed bf16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2));
}

__device__ __forceinline__ float pair16(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? max2f(a, b) : a + b;
}
__device__ __forceinline__ float pair32(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? max2f(a, b) : a + b;
}

// ---- multi-token form: records staged once per workgroup ---------------------
// From 64 query rows on, the latent records of each 32-key block are
// dequantised ONCE per workgroup into LDS as bf16 key rows (512 latent
// values, code x block scale, exact for the record's power-of-two scales,
// then the 64 bf16 rope values), in a ring of three stages. Both MFMA
// operands come from there:
//  * QK^T reads 16-byte pieces of the key rows (keys on M, two 16-key tiles);
//  * PV reads V^T straight from the same rows with the LDS transpose load
//    (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
//    i % 4 of the 8-byte reads of lanes i/4 + 4k (k = 0..3), so when lane j of
//    group g4 reads V[key k0 + 4 g4 + j/4][d + 4 (j % 4) ..], lane i holds
//    V[keys k0 + 4 g4 .. +3][d + i]. Two such reads (k0 = 0 and 16) give the
//    8 keys of a 16x16x32 A operand in the order in which the QK^T
//    accumulators hold the keys (4 g4 + i of each tile).
// Four waves, one per SIMD, each with all 64 query rows of the workgroup
// (four 16-row N blocks, so every K or V^T piece read from LDS feeds four
// MFMAs) and one head-dim quarter q: latent block q for QK^T (a partial S)
// and for PV (d_v 128 q .. 128 q + 127, its share of O), plus one of the
// four (16-key tile, rope k-step) pairs. One wave per SIMD has the whole
// register file (O alone is 128 registers). Against eight waves of 32 rows
// that read every piece twice (two per SIMD, same box): 4-6% faster.
// Per 32-key block the four waves write their partial S to LDS; after a
// barrier wave q owns rows 16 q .. 16 q + 15: it adds the four partials of
// those rows in a fixed order (each lane holds its row's keys
// 16 tt + 4 g4 + i, the QK^T accumulator layout), masks them and runs their
// softmax alone, and writes P as bf16, which in that layout is already the
// PV operand of its row block; after a second barrier every wave reads P of
// all 64 rows for its PV.
// With one wave per SIMD nothing overlaps a wave's phases but its own
// instruction order, so a step's MFMA work is one basic block: PV of the
// previous block, the next block's stage pieces, the loads of a later one,
// and QK^T of this one.
// The 256 threads split a block's loads (the key t >> 3: 16 latent bytes of
// each 128-value block, 16 rope bytes and the key's 16 scale bytes each),
// RING blocks ahead of the math in a register ring. The partial-S and P
// areas are single: each is rewritten only after the barrier that ends the
// reads of its previous contents.
constexpr int kLdsWaves = 4;
constexpr int kLdsRows = 64;                            // query rows per workgroup
constexpr int kLdsRb = kLdsRows / 16;                   // 16-row blocks per wave
constexpr int kStageKeys = 32;                          // keys per step
// bf16 key row + 32 B: rows sit 8 banks apart, and the 16-byte pieces of rows
// 4..7 (mod 8) are swapped in pairs (piece q -> q ^ 1), so 8 rows read at one
// column (the QK^T pieces) and 4 rows read 32 contiguous bytes each (the
// transpose loads) both hit distinct banks
constexpr int kKRowBytes = 2 * (kLatent + kRope) + 32;
constexpr int kStageBytes = kStageKeys * kKRowBytes;
constexpr int kStages = 3;
constexpr int kSpWaveBytes = 2 * kLdsRb * 64 * 16;              // partial S of a wave: [tt][rb][lane] f32x4
constexpr int kSpOffset = kStages * kStageBytes;
constexpr int kPOffset = kSpOffset + kLdsWaves * kSpWaveBytes;  // P: [rb][lane] 8 bf16
constexpr int kStatOffset = kPOffset + kLdsRb * 64 * 16;        // (max, sum) of the 64 rows
constexpr int kFlagOffset = kStatOffset + kLdsRows * 8;          // restart flag (int)
constexpr int kLdsBytes = kFlagOffset + 16;
static_assert(kLdsBytes <= 160 * 1024, "one workgroup's LDS must fit the CU's 160 KB");
constexpr float kFixedLog2 = 32.0f;  // p = exp2((s - m_run) c2) stays below 2^32
constexpr int kQkAhead = 3;          // K pieces read ahead of their MFMAs (source order)
constexpr int kPvAhead = 3;          // V^T tiles read ahead of their MFMAs (source order)

// One thread's loads of one 32-key block: key t >> 3, latent bytes
// 16 (t & 7) + 128 i (lat[i] lies in latent block i), rope bytes 16 (t & 7),
// and the key's four block scales (fp32 bits).
struct RawPiece {
  uint4 lat[4];
  uint4 rope;
  uint4 scl;
};

// Byte offset of byte `lane_off + c` of key row `row` in a stage (see
// kKRowBytes) is krow_base(row, lane_off) + c for every c whose bit 4 is
// clear (all the constant parts of the offsets below are multiples of 16).
__device__ __forceinline__ int krow_base(int row, int lane_off) {
  return row * kKRowBytes + (lane_off ^ (((row >> 2) & 1) << 4));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) uint8_t*)p);
}

// max / sum over the four lanes r16 + 16 g4 (a row's lanes in the
// accumulator layout)
__device__ __forceinline__ float max_over4(float x) { return pair32(pair16(x, true), true); }
__device__ __forceinline__ float sum_over4(float x) { return pair32(pair16(x, false), false); }

PKV_STAMP_STORAGE

// first_item: the workgroup's first work item (only it records stamps, in
// stamped builds)
template <bool CAUSAL_TAIL, int RING>
__device__ __forceinline__ void mla_lds_item(const MlaParams& p, int item, int tile, uint8_t* lds, bool first_item) {
  const int t = threadIdx.x;
  const int q = __builtin_amdgcn_readfirstlane(t >> 6);  // wave = head-dim quarter (wave-uniform)
  const int lane = t & 63;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  const int4 wk = p.work[item];
  const int b = wk.x;
  // tile ranges (one-wave plan): an empty range is padding; key ranges
  // (balanced plan): an empty range is the item of an empty sequence, whose
  // rows still get O = 0, LSE = -inf
  const bool empty = p.bin_offsets ? wk.z < wk.y : wk.z <= wk.y;
  if (empty || b < 0 || b >= p.num_seqs) return;  // the whole workgroup returns
  const int ns = p.n_splits[b];
  const bool direct = ns <= 1;
  const int slot = wk.w;
  if (!direct && (slot < 0 || slot >= p.max_splits)) return;

  const int page_size = 1 << p.page_shift;
  int L = p.seq_lens[b];
  L = max(0, min(L, p.max_blocks * page_size));
  const int k_begin = p.bin_offsets ? wk.y : wk.y * kTileKeys;
  const int k_end = min(p.bin_offsets ? wk.z : wk.z * kTileKeys, L);

  // rows in the MFMA layout: n = row0 + 16 rb + r16; rows past the last run
  // like the others (on zero query rows) and write nothing
  const int row0 = tile * kLdsRows;
  int qtok[kLdsRb], qhead[kLdsRb];
  bool row_ok[kLdsRb];
  for (int rb = 0; rb < kLdsRb; ++rb) {
    const int n = row0 + 16 * rb + r16;
    row_ok[rb] = n < p.rows;
    const int qi = n / p.h_q;
    qtok[rb] = b * p.q_len + qi;
    qhead[rb] = n - qi * p.h_q;
  }
  // the row this wave owns in the softmax: row block q, row r16; this lane
  // holds its keys 16 tt + 4 g4 + i
  const int on = min(row0 + 16 * q + r16, p.rows - 1);
  const int olim = min(CAUSAL_TAIL ? L - p.q_len + on / p.h_q : L - 1, k_end - 1);
  const int on_min = min(row0 + 16 * q, p.rows - 1);  // first row this wave owns
  const int olim_min = min(CAUSAL_TAIL ? L - p.q_len + on_min / p.h_q : L - 1, k_end - 1);
  const float c2 = p.scale_log2e;

  // Q as the B operand of this wave's quarter of d_qk: k-step k < 4 holds
  // q[n][128 q + 32 k + 8 g4 .. +7] (latent block q), k = 4 rope k-step q & 1
  bf16x8 qv[kLdsRb][5];
  for (int rb = 0; rb < kLdsRb; ++rb) {
    const uint8_t* qrow = p.q + (int64_t)qtok[rb] * p.q_tok + (int64_t)qhead[rb] * p.q_head;
    for (int k = 0; k < 5; ++k) {
      const int d = k < 4 ? 128 * q + 32 * k + 8 * g4 : kLatent + 32 * (q & 1) + 8 * g4;
      if (row_ok[rb]) {
        qv[rb][k] = *reinterpret_cast<const bf16x8*>(qrow + 2 * d);
      } else {
        for (int e = 0; e < 8; ++e) qv[rb][k][e] = (__bf16)0.0f;
      }
    }
  }

  f32x4 oacc[kLdsRb][8];  // [row block][16-row tile mt]: O^T[128 q + 16 mt + 4 g4 + i][row 16 rb + r16]
  // m_run: the reference max (raw-score units) of the owned row, set by the
  // row's first visible block and then fixed, so O is never rescaled inside
  // the loop. P = exp2((s - m_run) c2) may grow up to 2^kFixedLog2, which
  // bf16 P and the fp32 sums absorb. m_seen: the largest score this lane has
  // seen. l_part: this lane's share of the row sum.
  float m_run = -INFINITY, m_seen = -INFINITY, l_part;
  // an LDS pointer (a generic one would make these FLAT accesses, whose waits
  // also wait for every global load in flight)
  volatile __attribute__((address_space(3))) int* restart_flag =
      (volatile __attribute__((address_space(3))) int*)((__attribute__((address_space(3))) uint8_t*)lds + kFlagOffset);
  auto barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  bool again;
  // A block with a score that would put its p past 2^kFixedLog2 (scores
  // rising that far after a row's first visible block: pathological inputs
  // only) sets the flag; the waves read it after the second barrier of every
  // sixth block and after the last, all at the same point, and the workgroup
  // runs the item again from its first key with each row's reference at the
  // largest score seen. Each run gets further than the one before (the
  // blocks it has seen can no longer pass the bound), so the runs end.
  do {
  again = false;
  l_part = 0.f;
  for (int rb = 0; rb < kLdsRb; ++rb)
    for (int mt = 0; mt < 8; ++mt) oacc[rb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (k_end > k_begin) {
    const int32_t* bt = p.block_table + (int64_t)b * p.bt_row;
    const int last_key = k_end - 1;
    const int pmask = page_size - 1;
    // pages of a 32-key block's two 16-key halves (page_size >= 16), read
    // with scalar loads through the constant address space: their waits count
    // no vector loads, so none of them waits for the KV loads in flight
    struct Pages {
      int h0, h1;
    };
    auto page_pair = [&](int kb) -> Pages {
      const __attribute__((address_space(4))) int32_t* cbt = (const __attribute__((address_space(4))) int32_t*)bt;
      return Pages{cbt[min(kb, last_key) >> p.page_shift], cbt[min(kb + 16, last_key) >> p.page_shift]};
    };
    auto clamp_page = [&](int pg) -> int { return min(max(pg, 0), p.num_pages - 1); };

    // fetch u: the loads of block k_begin + 32u into ring slot u % RING, with
    // the pages from page slot u % 3 (loaded two fetches earlier); it loads
    // the pages of fetch u + 2. Waves 0-1 load keys 0-15, waves 2-3 keys
    // 16-31, so each wave reads one page per load.
    Pages pv[3];
    pv[0] = page_pair(k_begin);
    pv[1] = page_pair(k_begin + kStageKeys);
    const int my_key = t >> 3, part = t & 7;
    // A load's address is the wave-uniform page base (scalar registers) plus a
    // 32-bit lane offset: the key's row inside the page times the row stride
    // (page_size * row stride < 2^30, as the host checks) plus the lane's
    // bytes in the row.
    auto fetch = [&](RawPiece& r, int kb, const int ps) {
      const int64_t pgk = clamp_page((q >> 1) ? pv[ps].h1 : pv[ps].h0);
      const uint32_t key = (uint32_t)(min(kb + my_key, last_key) & pmask);
      const uint8_t* lat = p.lat + pgk * p.lat_page;
      const uint8_t* rope = p.rope + pgk * p.rope_page;
      const uint8_t* scl = p.scl + pgk * p.scl_page;
      const uint32_t lat_off = key * (uint32_t)p.lat_row + 16u * part;
      for (int i = 0; i < 4; ++i) r.lat[i] = *reinterpret_cast<const uint4*>(lat + (lat_off + 128u * i));
      r.rope = *reinterpret_cast<const uint4*>(rope + (key * (uint32_t)p.rope_row + 16u * part));
      r.scl = *reinterpret_cast<const uint4*>(scl + key * (uint32_t)p.scl_row);
      pv[(ps + 2) % 3] = page_pair(kb + 2 * kStageKeys);
    };
    // The key row's bf16 latent values 128 i + 16 part .. +15 (pieces 2 i and
    // 2 i + 1 of this thread, 16 bytes each), then its rope bytes 16 part
    // (piece 8). The power-of-two form (the record format: the scaled convert
    // is exact) is always converted and written; a wave with a key whose
    // scales are not all powers of two then rewrites the block's pieces with
    // the fp32 product (a uniform branch after the writes, so the common path
    // is one basic block with the MFMAs it is interleaved with).
    auto convert = [&](const RawPiece& r, bf16x8 (&c)[8]) {
      const float sc[4] = {__uint_as_float(r.scl.x), __uint_as_float(r.scl.y), __uint_as_float(r.scl.z),
                           __uint_as_float(r.scl.w)};
      for (int i = 0; i < 4; ++i) {
        c[2 * i] = e4m3x8_times_pow2(half_of(r.lat[i], 0), sc[i]);
        c[2 * i + 1] = e4m3x8_times_pow2(half_of(r.lat[i], 1), sc[i]);
      }
    };
    auto piece_at = [&](uint8_t* st, int k) -> uint8_t* {
      return st + (k < 8 ? krow_base(my_key, 256 * (k >> 1) + 32 * part + 16 * (k & 1))
                         : krow_base(my_key, 2 * kLatent + 16 * part));
    };
    auto write_piece = [&](uint8_t* st, const RawPiece& r, const bf16x8 (&c)[8], int k) {
      if (k < 8)
        *reinterpret_cast<bf16x8*>(piece_at(st, k)) = c[k];
      else
        *reinterpret_cast<uint4*>(piece_at(st, 8)) = r.rope;
    };
    auto stage_fixup = [&](const RawPiece& r, uint8_t* st) {
      if (__builtin_amdgcn_ballot_w64(!pow2_scales(r.scl)) != 0) {
        const float sc[4] = {__uint_as_float(r.scl.x), __uint_as_float(r.scl.y), __uint_as_float(r.scl.z),
                             __uint_as_float(r.scl.w)};
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<bf16x8*>(piece_at(st, 2 * i)) = e4m3x8_times_any(half_of(r.lat[i], 0), sc[i]);
          *reinterpret_cast<bf16x8*>(piece_at(st, 2 * i + 1)) = e4m3x8_times_any(half_of(r.lat[i], 1), sc[i]);
        }
      }
    };

    // this lane's QK^T piece (key row r16 of a tile, bytes 16 g4 ..) and
    // transpose-read piece (key row 4 g4 + r16 / 4, bytes 8 (r16 % 4) ..);
    // rows 16 apart share the swizzle
    const int qk_base = krow_base(r16, 16 * g4);
    const int tr_base = krow_base(4 * g4 + (r16 >> 2), 8 * (r16 & 3));
    // Each wave takes one of the four (tile, rope k-step) pairs: rope k-step
    // q & 1 on tile tr = q >> 1, so every wave runs 36 QK^T MFMAs. It runs
    // the other tile first (four latent k-steps), then tile tr (four latent
    // k-steps and its rope step); piece i of that sequence:
    const int tr_tile = q >> 1;
    auto qk_piece = [&](const uint8_t* st, int i) -> bf16x8 {
      const int tt = i < 4 ? 1 - tr_tile : tr_tile;
      const int off = i < 8 ? 2 * (128 * q + 32 * (i & 3)) : 2 * (kLatent + 32 * (q & 1));
      return *reinterpret_cast<const bf16x8*>(st + qk_base + tt * 16 * kKRowBytes + off);
    };
    uint8_t* const sp_own = lds + kSpOffset + q * kSpWaveBytes;
    auto put_s = [&](int tt, const f32x4 (&s)[kLdsRb]) {
      for (int rb = 0; rb < kLdsRb; ++rb)
        *reinterpret_cast<f32x4*>(sp_own + ((kLdsRb * tt + rb) * 64 + lane) * 16) = s[rb];
    };
    // partial S (sa: the first tile, sb: tile tr; S[key 16 tt + 4 g4 + i][row
    // 16 rb + r16]) of the block in stage st over this wave's quarter of
    // d_qk, written to this wave's partial-S area ([tt][rb][lane]); each K
    // piece is read kQkAhead pieces ahead of its four MFMAs; both tiles'
    // partial S are stored after the last MFMA is issued (stored under the
    // second tile's first k-step, the first tile's delayed the K reads queued
    // behind it: T = 16 256.4 -> 253.8 us). The next block's rope piece is
    // staged at the start.
    auto qk_quarter = [&](const uint8_t* st, uint8_t* st_next, const RawPiece& nr, const bf16x8 (&nc)[8]) {
      f32x4 sa[kLdsRb], sb[kLdsRb];
      bf16x8 pa[kQkAhead + 1];
      for (int i = 0; i < kQkAhead; ++i) pa[i] = qk_piece(st, i);
      write_piece(st_next, nr, nc, 8);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        if (i + kQkAhead < 9) pa[(i + kQkAhead) % (kQkAhead + 1)] = qk_piece(st, i + kQkAhead);
        const bf16x8 k_op = pa[i % (kQkAhead + 1)];
        for (int rb = 0; rb < kLdsRb; ++rb) {
          const bf16x8 q_op = qv[rb][i < 8 ? (i & 3) : 4];
          if (i < 4)
            sa[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_op, q_op, i == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sa[rb],
                                                             0, 0, 0);
          else
            sb[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_op, q_op, i == 4 ? f32x4{0.f, 0.f, 0.f, 0.f} : sb[rb],
                                                             0, 0, 0);
        }
      }
      put_s(1 - tr_tile, sa);
      put_s(tr_tile, sb);
    };
    // S of the owned row at this lane's keys of both tiles: the partials of
    // waves 0 .. 3 added in that order, masked
    const uint8_t* const sp_row = lds + kSpOffset + (q * 64 + lane) * 16;
    auto own_s = [&](int kb, f32x4 (&sv)[2]) {
      f32x4 a[2][4];
      for (int tt = 0; tt < 2; ++tt)
        for (int w = 0; w < 4; ++w)
          a[tt][w] = *reinterpret_cast<const f32x4*>(sp_row + w * kSpWaveBytes + tt * kLdsRb * 64 * 16);
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 s = a[tt][0] + a[tt][1];
        s += a[tt][2];
        s += a[tt][3];
        sv[tt] = s;
      }
      if (kb + kStageKeys - 1 > olim_min) {
        for (int tt = 0; tt < 2; ++tt)
          for (int i = 0; i < 4; ++i)
            if (kb + 16 * tt + 4 * g4 + i > olim) sv[tt][i] = -INFINITY;
      }
    };
    // softmax of the owned row for this block: the reference (only while
    // some row of the wave has none yet, the row max over its four lanes),
    // eight exponentials, P to the PV operand area of row block q
    uint8_t* const p_out = lds + kPOffset + (q * 64 + lane) * 16;
    auto softmax_own = [&](const f32x4 (&s)[2], bool& overflow) {
      const float mx = max3f(max3f(s[0][0], s[0][1], s[0][2]), max3f(s[0][3], s[1][0], s[1][1]),
                             max3f(s[1][2], s[1][3], -INFINITY));
      m_seen = max2f(m_seen, mx);
      if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY)) {
        // the first visible block sets the reference (O and l are still zero)
        const float row_mx = max_over4(mx);
        m_run = m_run == -INFINITY ? row_mx : m_run;
      }
      overflow = (mx - m_run) * c2 > kFixedLog2;
      // one fma per score: exp2(s c2 - m c2); no visible key yet: exp2(-inf) = 0
      const float off = m_run == -INFINITY ? 0.f : -m_run * c2;
      float pr[8];
      for (int tt = 0; tt < 2; ++tt)
        for (int i = 0; i < 4; ++i) pr[4 * tt + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][i], c2, off));
      l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
      *reinterpret_cast<uint4*>(p_out) = uint4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                               pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
    };
    // O^T += V^T P^T for this wave's 128 d_v: V^T tile mt read kPvAhead tiles
    // ahead of its four MFMAs
    auto v_tile = [&](const uint8_t* st, int mt) -> bf16x8 {
      const uint8_t* v = st + tr_base + 2 * (128 * q + 16 * mt);
      const s16x4 lo = lds_read_tr16(v);
      const s16x4 hi = lds_read_tr16(v + 16 * kKRowBytes);
      const s16x8 a16 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      bf16x8 a;
      __builtin_memcpy(&a, &a16, 16);
      return a;
    };
    const uint8_t* const p_in = lds + kPOffset + lane * 16;
    // PV of the block in stage st; when given the next block's converted
    // pieces, they are written to st_next after PV's MFMAs are issued (the
    // LDS serves a wave's accesses in order, so stores placed between the
    // MFMAs delayed the V^T and K reads behind them: T = 16 261.7 -> 256.7
    // us, T = 8 142.0 -> 138.8 against one store after each V^T tile)
    auto pv_quarter = [&](const uint8_t* st, uint8_t* st_next, const RawPiece* nr, const bf16x8 (*nc)[8]) {
      u32x4 pb[kLdsRb];
      for (int rb = 0; rb < kLdsRb; ++rb) pb[rb] = *reinterpret_cast<const u32x4*>(p_in + rb * 64 * 16);
      bf16x8 va[kPvAhead + 1];
      for (int i = 0; i < kPvAhead; ++i) va[i] = v_tile(st, i);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (mt + kPvAhead < 8) va[(mt + kPvAhead) % (kPvAhead + 1)] = v_tile(st, mt + kPvAhead);
        for (int rb = 0; rb < kLdsRb; ++rb)
          oacc[rb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mt % (kPvAhead + 1)],
                                                                __builtin_bit_cast(bf16x8, pb[rb]), oacc[rb][mt], 0, 0, 0);
      }
      if (nc)
        for (int k = 0; k < 8; ++k) write_piece(st_next, *nr, *nc, k);
    };

    // Two barriers per step. Block j: fetched in step j - RING, converted and
    // staged into stage (j % 3) in step j - 1. Step j: PV of block j - 1,
    // the loads of block j + RING, QK^T of block j with its partial S
    // written, block j + 1's pieces written between them (one basic block),
    // B1; the owners reduce, run the softmax and write P, B2. Stage j is
    // read by QK^T in step j and by PV in step j + 1 and rewritten in step
    // j + 2, after the barriers of step j + 1. Step 0 has no PV; rounds of 6
    // steps from step 1 on keep the ring and stage indices compile-time; PV
    // of the last block follows the loop.
    static_assert(RING == 2, "the step indices below assume two blocks in flight");
    constexpr int kRound = 6;
    const int nblocks = (k_end - k_begin + kStageKeys - 1) / kStageKeys;
    RawPiece ring[RING];
    bf16x8 nc[8];
    fetch(ring[0], k_begin, 0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(ring[1], k_begin + kStageKeys, 1);
    __builtin_amdgcn_sched_barrier(0);
    convert(ring[0], nc);
    for (int k = 0; k < 9; ++k) write_piece(lds, ring[0], nc, k);
    stage_fixup(ring[0], lds);
    barrier();
    auto softmax_step = [&](int kb) {
      f32x4 sv[2];
      own_s(kb, sv);
      bool overflow;
      softmax_own(sv, overflow);
      if (__builtin_amdgcn_ballot_w64(overflow) && lane == 0) *restart_flag = 1;
    };
    // step 0
    {
      fetch(ring[0], k_begin + RING * kStageKeys, 2);
      convert(ring[1], nc);
      for (int k = 0; k < 8; ++k) write_piece(lds + kStageBytes, ring[1], nc, k);
      qk_quarter(lds, lds + kStageBytes, ring[1], nc);
      stage_fixup(ring[1], lds + kStageBytes);
      barrier();
      softmax_step(k_begin);
      barrier();
    }
    const int rounds = (nblocks - 1 + kRound - 1) / kRound;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int s = 0; s < kRound; ++s) {
        const int j = r * kRound + s + 1;
        if (j >= nblocks) goto loop_done;
        const int kb = k_begin + j * kStageKeys;
        RawPiece& nr = ring[s & 1];  // block j + 1
        uint8_t* const st_prev = lds + (s % 3) * kStageBytes;
        uint8_t* const st_cur = lds + ((s + 1) % 3) * kStageBytes;
        uint8_t* const st_next = lds + ((s + 2) % 3) * kStageBytes;
        // stamps (stamped builds): load issue + conversion 0 -> 1, MFMA phase
        // 1 -> 2, first barrier 2 -> 3, softmax 3 -> 4, second barrier 4 -> 5
        PKV_STAMP_VARS
        PKV_STAMP(0);
        fetch(ring[(s + 1) & 1], kb + RING * kStageKeys, s % 3);
        convert(nr, nc);
        PKV_STAMP(1);
        pv_quarter(st_prev, st_next, &nr, &nc);
        qk_quarter(st_cur, st_next, nr, nc);
        stage_fixup(nr, st_next);
        PKV_STAMP(2);
        barrier();
        PKV_STAMP(3);
        softmax_step(kb);
        PKV_STAMP(4);
        barrier();
        PKV_STAMP(5);
        PKV_STAMP_SAVE(j, first_item);
        // the flag is read once per round: a block past the bound only fills
        // O, l and P with values the restart throws away
        if (s == kRound - 1 && __builtin_amdgcn_readfirstlane(*restart_flag)) {
          again = true;
          goto item_end;
        }
      }
    }
  loop_done:
    if (__builtin_amdgcn_readfirstlane(*restart_flag)) {
      again = true;
    } else {
      const int jl = nblocks - 1;
      pv_quarter(lds + (jl % 3) * kStageBytes, nullptr, nullptr, nullptr);
    }
  }
item_end:
  if (again) {
    barrier();  // every wave has read the flag
    if (t == 0) *restart_flag = 0;
    m_run = max_over4(m_seen);
  }
  } while (again);

  // ---- epilogue: the owners publish each row's (max, sum); every wave
  // writes its d_v quarter of O; LSE / (max, sum) from quarter 0
  const float l_row = sum_over4(l_part);
  float2* const stat = reinterpret_cast<float2*>(lds + kStatOffset);
  if (g4 == 0) stat[16 * q + r16] = float2{m_run == -INFINITY ? -INFINITY : m_run * p.scale, l_row};
  barrier();
  for (int rb = 0; rb < kLdsRb; ++rb) {
    if (!row_ok[rb]) continue;
    const float2 ml = stat[16 * rb + r16];
    const float m_nat = ml.x, l = ml.y;
    const int64_t stat_row = (int64_t)b * p.rows + row0 + 16 * rb + r16;
    const int d0 = 128 * q + 4 * g4;
    if (direct) {
      const float inv = l > 0.f ? p.o_scale / l : 0.f;
      uint8_t* orow_p = p.o + (int64_t)qtok[rb] * p.o_tok + (int64_t)qhead[rb] * p.o_head;
      for (int mt = 0; mt < 8; ++mt) {
        bf16x4 out;
        for (int i = 0; i < 4; ++i) out[i] = (__bf16)(oacc[rb][mt][i] * inv);
        *reinterpret_cast<bf16x4*>(orow_p + 2 * (d0 + 16 * mt)) = out;
      }
      if (q == 0 && g4 == 0) p.lse[stat_row] = l > 0.f ? m_nat + logf(l) : -INFINITY;
    } else {
      const int64_t prow = (int64_t)slot * p.num_seqs * p.rows + stat_row;
      float* dst = p.ws_o + prow * kDv + d0;
      for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(dst + 16 * mt) = oacc[rb][mt];
      if (q == 0 && g4 == 0) p.ws_ml[prow] = float2{m_nat, l};
    }
  }
}

// XCD-aware grid: the workgroups of one work item's q-row tiles read the same
// records, so they are placed on one XCD (sharing its L2) at about the same
// time. Workgroups are dispatched to the 8 XCDs round robin, so ids i, i + 8,
// i + 16, ... share an XCD: a chunk of 8 * tiles consecutive ids holds 8
// items x tiles, with the item varying fastest (the last chunk holds what is
// left).
constexpr int kXcds = 8;

__device__ __forceinline__ void xcd_item_tile(int id, int units, int tiles, int& unit, int& tile) {
  const int chunk = id / (kXcds * tiles);
  const int local = id - chunk * kXcds * tiles;
  const int left = min(kXcds, units - chunk * kXcds);
  unit = chunk * kXcds + local % left;
  tile = local / left;
}

constexpr int kLdsRing = 2;  // raw blocks in flight per thread

template <bool CAUSAL_TAIL>
__global__ __launch_bounds__(64 * kLdsWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_lds_kernel(MlaParams p, int units, int tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_stage_lds[];
  if (threadIdx.x == 0) *reinterpret_cast<int*>(mla_stage_lds + kFlagOffset) = 0;
  __syncthreads();
  int unit, tile;
  xcd_item_tile(blockIdx.x, units, tiles, unit, tile);
  int it = unit, it_end = unit + 1;
  if (p.bin_offsets) {
    it = p.bin_offsets[unit];
    it_end = p.bin_offsets[unit + 1];
  }
#if PKV_STAMPS
  const int it0 = it;
#define PKV_FIRST_ITEM (it == it0)
#else
#define PKV_FIRST_ITEM true
#endif
  for (; it < it_end; ++it) {
    mla_lds_item<CAUSAL_TAIL, kLdsRing>(p, it, tile, mla_stage_lds, PKV_FIRST_ITEM);
    __syncthreads();  // the next item's first stage overwrites LDS
  }
#undef PKV_FIRST_ITEM
}

// ---- pair form: fewer than 64 query rows -------------------------------------
// Two waves per 16-row group split every record: wave h (HALF) takes latent
// blocks 2h and 2h + 1 (d_v 256 h .. 256 h + 255) and rope k-step h. It loads
// only those bytes, converts its latent codes to bf16 once (the QK^T operand,
// also stored to its LDS rows, from which the V^T operand is read back with
// the transpose load, see the staged form) and computes the partial S over
// its part of d_qk. The pair swaps partial S through LDS (one barrier per
// block); both add the two parts in the same order, so they hold identical S
// and softmax statistics. O: 256 d_v x 16 rows = 64 VGPRs per lane, so two
// waves fit on a SIMD. One or two row groups per workgroup.
constexpr int kPairMaxGroups = 2;
constexpr int kPairStages = 4;  // ring of 16-key blocks: three in flight while one is processed
constexpr int kPairQSteps = 9;  // 8 latent k-steps + 1 rope k-step
constexpr int kHalfRowBytes = 2 * (kDv / 2) + 32;  // bf16 half row + 32 B, swizzled as the staged rows
constexpr int kPairV = kPairQSteps * 64 * 16;      // after the parked query
constexpr int kPairScl = kPairV + kBlockKeys * kHalfRowBytes;
constexpr int kPairX = kPairScl + kBlockKeys * 8;  // partial S, two slots (block parity)
constexpr int kPairWaveBytes = kPairX + 2 * 64 * 16;

struct HalfRec {
  uint4 kl[2][2];  // key kb + r16: latent bytes 128 (2 HALF + j) + 64 h + 16 g4 .. +15
  uint4 kr;        // key kb + r16: rope values 32 HALF + 8 g4 .. +7
  float2 sc;       // key kb + r16: block scales 2 HALF, 2 HALF + 1
};

__device__ __forceinline__ int hrow_base(int row, int lane_off) {
  return row * kHalfRowBytes + (lane_off ^ (((row >> 2) & 1) << 4));
}

template <bool CAUSAL_TAIL, int HALF>
__device__ __forceinline__ void mla_pair_item(const MlaParams& p, int item, int tile, int groups, uint8_t* lds,
                                              bool first_item) {
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int grp = w >> 1;

  const int4 wk = p.work[item];
  const int b = wk.x;
  // an empty key range (balanced plan) is an empty sequence's item: its rows
  // still get their output; an empty tile range is padding
  const bool empty = p.bin_offsets ? wk.z < wk.y : wk.z <= wk.y;
  if (empty || b < 0 || b >= p.num_seqs) return;  // the whole workgroup returns
  const int k_begin = p.bin_offsets ? wk.y : wk.y * kTileKeys;
  const int k_plan = p.bin_offsets ? wk.z : wk.z * kTileKeys;  // planned end: lengths of the plan are upper bounds
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_row;

  // Start-up: the block-table entries of the first fetches, the query, the
  // split count and the sequence length are independent loads, issued
  // together (one round trip where a dependent chain takes three). The
  // entries are those of the planned chunk; when the runtime length ends the
  // chunk before the last of them, they are loaded again below.
  constexpr int kPageAhead = kPairStages - 1;
  int pv[kPairStages];
  for (int u = 0; u < kPageAhead; ++u)
    pv[u] = bt[min(min(k_begin + kBlockKeys * u, max(k_plan - 1, 0)) >> p.page_shift, p.max_blocks - 1)];

  // rows of this wave's group; a group past the last row still runs the loop
  // (on a zero query) and meets every barrier
  const int row0 = (tile * groups + grp) * 16;
  const int n = row0 + r16;
  const bool row_ok = n < p.rows;
  const int qi = n / p.h_q;
  const int qtok = b * p.q_len + qi;
  const int qhead = n - qi * p.h_q;
  // this wave's part of the query as the QK^T B operand (k-steps of its two
  // latent blocks, same head-dim permutation as the K loads, then its rope
  // k-step), parked in LDS below; only this wave reads it. Rows past the last
  // load the last row (no branch) and are zeroed.
  bf16x8 qreg[kPairQSteps];
  {
    const int nq = row_ok ? n : p.rows - 1;
    const int qiq = nq / p.h_q;
    const uint8_t* qrow = p.q + (int64_t)(b * p.q_len + qiq) * p.q_tok + (int64_t)(nq - qiq * p.h_q) * p.q_head;
    for (int k = 0; k < kPairQSteps; ++k) {
      const int blk = 2 * HALF + (k >> 2), s = k & 3;
      const int d = k < 8 ? 128 * blk + 64 * (s >> 1) + 16 * g4 + 8 * (s & 1) : kLatent + 32 * HALF + 8 * g4;
      qreg[k] = *reinterpret_cast<const bf16x8*>(qrow + 2 * d);
    }
  }
  const int ns = p.n_splits[b];
  int L = p.seq_lens[b];
  if (!row_ok)
    for (int k = 0; k < kPairQSteps; ++k)
      for (int e = 0; e < 8; ++e) qreg[k][e] = (__bf16)0.0f;

  const bool direct = ns <= 1;
  const int slot = wk.w;
  if (!direct && (slot < 0 || slot >= p.max_splits)) return;
  const int page_size = 1 << p.page_shift;
  L = max(0, min(L, p.max_blocks * page_size));
  const int k_end = min(k_plan, L);
  const int lim = min(CAUSAL_TAIL ? L - p.q_len + qi : L - 1, k_end - 1);
  const int qi_min = min(row0, p.rows - 1) / p.h_q;
  const int lim_min = min(CAUSAL_TAIL ? L - p.q_len + qi_min : L - 1, k_end - 1);
  const float c2 = p.scale_log2e;

  uint8_t* const wl = lds + w * kPairWaveBytes;
  uint8_t* const xl = lds + (w ^ 1) * kPairWaveBytes + kPairX;  // the partner's partial S
  bf16x8(*qw)[64] = reinterpret_cast<bf16x8(*)[64]>(wl);
  for (int k = 0; k < kPairQSteps; ++k) qw[k][lane] = qreg[k];

  f32x4 oacc[2][8];  // [block j][16-row tile mt]: O^T[256 HALF + 128 j + 16 mt + 4 g4 + i][n]
  for (int j = 0; j < 2; ++j)
    for (int mt = 0; mt < 8; ++mt) oacc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  if (k_end > k_begin) {
    const int last_key = k_end - 1;
    const int pmask = page_size - 1;
    auto page_of = [&](int kb) -> int { return bt[min(kb, last_key) >> p.page_shift]; };
    auto clamp_page = [&](int pg) -> int { return min(max(pg, 0), p.num_pages - 1); };
    // the early entries are right unless the chunk ends before the last of them
    if (k_begin + kBlockKeys * (kPageAhead - 1) > last_key)
      for (int u = 0; u < kPageAhead; ++u) pv[u] = page_of(k_begin + kBlockKeys * u);
    auto load_block = [&](int kb, int pg) {
      HalfRec r;
      // page bases are wave-uniform (scalar); a lane's row offset fits 32 bits
      // (page_size * row stride < 2^30, checked on the host), so each load is
      // a scalar base plus one 32-bit offset and an immediate
      const uint32_t row = (uint32_t)(min(kb + r16, last_key) & pmask);
      const uint8_t* lat = p.lat + (int64_t)pg * p.lat_page;
      const uint8_t* rope = p.rope + (int64_t)pg * p.rope_page;
      const uint8_t* scl = p.scl + (int64_t)pg * p.scl_page;
      const uint8_t* lr = lat + (row * (uint32_t)p.lat_row + 16u * (uint32_t)g4);
      for (int j = 0; j < 2; ++j)
        for (int h = 0; h < 2; ++h) r.kl[j][h] = *reinterpret_cast<const uint4*>(lr + (256 * HALF + 128 * j + 64 * h));
      r.kr = *reinterpret_cast<const uint4*>(rope + (row * (uint32_t)p.rope_row + 16u * (uint32_t)g4) + 64 * HALF);
      r.sc = *reinterpret_cast<const float2*>(scl + row * (uint32_t)p.scl_row + 8 * HALF);
      return r;
    };
    // page ring: fetch u reads slot u % kPairStages and loads the page of
    // fetch u + kPageAhead into the slot fetch u - 1 used. Loads complete in
    // order, so the wait for that page must not come before the data of
    // fetch u - 1 is due anyway: a shorter page distance would cut the ring.
    auto fetch = [&](HalfRec& r, int kb, const int s) {
      const int pg = clamp_page(__builtin_amdgcn_readlane(pv[s], 0));
      r = load_block(kb, pg);
      pv[(s + kPageAhead) % kPairStages] = page_of(kb + kPageAhead * kBlockKeys);
    };

    // this lane's transpose-read piece: key row 4 g4 + r16 / 4, bytes 8 (r16 % 4) ..
    const int tr_base = hrow_base(4 * g4 + (r16 >> 2), 8 * (r16 & 3));
    // stamps (stamped builds): issue 0 -> 1, wait for the block 1 -> 2, conversion and
    // partial S 2 -> 3, exchange barrier 3 -> 4, softmax 4 -> 5, PV 5 -> 6
    PKV_STAMP_VARS
    auto process = [&](const HalfRec& cur, int kb, const int xs) {
      asm volatile("" ::: "memory");
      // the four lanes of a key store the same scales (no branch: a divergent
      // store here costs the loop its load-wait precision)
      *reinterpret_cast<float2*>(wl + kPairScl + 8 * r16) = cur.sc;
      // ---- partial S over this wave's latent blocks and rope k-step ------------
      f32x4 acc[2];
      for (int j = 0; j < 2; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = e4m3x8_to_bf16(half_of(cur.kl[j][s >> 1], s & 1));
          *reinterpret_cast<bf16x8*>(wl + kPairV + hrow_base(r16, 32 * g4 + 16 * (s & 1)) + 256 * j +
                                     128 * (s >> 1)) = a;
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qw[4 * j + s][lane], acc[j], 0, 0, 0);
        }
      }
      const f32x4 accr =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.kr), qw[8][lane], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      // lane holds partial S[key kb + 4 g4 + i][row n]; other lanes' stores are
      // read back from here on
      asm volatile("" ::: "memory");
      float2 scl[4];
      for (int i = 0; i < 4; ++i) scl[i] = *reinterpret_cast<const float2*>(wl + kPairScl + 8 * (4 * g4 + i));
      f32x4 part;
      for (int i = 0; i < 4; ++i) part[i] = accr[i] + scl[i].x * acc[0][i] + scl[i].y * acc[1][i];
      *reinterpret_cast<f32x4*>(wl + kPairX + xs * 1024 + 16 * lane) = part;
      PKV_STAMP(3);
      __syncthreads();
      PKV_STAMP(4);
      const f32x4 other = *reinterpret_cast<const f32x4*>(xl + xs * 1024 + 16 * lane);
      float sv[4];
      for (int i = 0; i < 4; ++i) sv[i] = part[i] + other[i];  // the same sum in both waves
      if (kb + kBlockKeys - 1 > lim_min) {
        for (int i = 0; i < 4; ++i)
          if (kb + 4 * g4 + i > lim) sv[i] = -INFINITY;
      }
      // ---- online softmax (bf16 P: the reference max may lag) -----------------
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = pair32(pair16(mx, true), true);
      const float m_max = fmaxf(m_run, mx);
      const bool move = m_run == -INFINITY ? m_max != -INFINITY : (m_max - m_run) * c2 > kLazyLog2;
      const float m_new = move ? m_max : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      float pr[4], psum = 0.f;
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f((sv[i] - m_use) * c2);
        psum += pr[i];
      }
      l_part = l_part * corr + psum;
      if (__builtin_amdgcn_ballot_w64(move)) {
        for (int j = 0; j < 2; ++j)
          for (int mt = 0; mt < 8; ++mt) oacc[j][mt] *= corr;
      }
      m_run = m_new;
      PKV_STAMP(5);
      // ---- O^T += V^T (P * scale)^T for this wave's 256 d_v -------------------
      for (int j = 0; j < 2; ++j) {
        bf16x4 pb;  // P scaled by the block scale of latent block 2 HALF + j
        for (int i = 0; i < 4; ++i) pb[i] = (__bf16)(pr[i] * (j ? scl[i].y : scl[i].x));
        for (int mt = 0; mt < 8; ++mt) {
          const s16x4 t4 = lds_read_tr16(wl + kPairV + tr_base + 256 * j + 32 * mt);
          bf16x4 a;
          __builtin_memcpy(&a, &t4, 8);
          oacc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, oacc[j][mt], 0, 0, 0);
        }
      }
    };

    // Rounds of kPairStages blocks keep ring slots and exchange slots (block
    // parity) compile-time; blocks past the chunk load clamped rows and are
    // masked, so both waves of a pair run the same barriers.
    // The prologue issues its loads in loop order (no reordering across the
    // fences): the waits at the loop head serve both entry paths, so a
    // reshuffled prologue would make them wait for more than the oldest block.
    HalfRec ring[kPairStages];
#pragma unroll
    for (int s = 0; s < kPairStages - 1; ++s) {
      fetch(ring[s], k_begin + kBlockKeys * s, s);
      asm volatile("" ::: "memory");
    }
    const int rounds = (k_end - k_begin + kBlockKeys * kPairStages - 1) / (kBlockKeys * kPairStages);
    for (int r = 0; r < rounds; ++r) {
      const int kb0 = k_begin + r * kBlockKeys * kPairStages;
#pragma unroll
      for (int s = 0; s < kPairStages; ++s) {
        const int kb = kb0 + kBlockKeys * s;
        PKV_STAMP(0);
        fetch(ring[(s + kPairStages - 1) % kPairStages], kb + kBlockKeys * (kPairStages - 1),
              (s + kPairStages - 1) % kPairStages);
        PKV_STAMP(1);
#if PKV_STAMPS
        asm volatile("" ::"v"(ring[s].sc.x), "v"(ring[s].sc.y));  // the block's last load has landed
#endif
        PKV_STAMP(2);
        process(ring[s], kb, s & 1);
        PKV_STAMP(6);
        PKV_STAMP_SAVE(r * kPairStages + s, first_item);
      }
    }
  }

  // ---- epilogue: this wave's d_v half; LSE / (max, sum) from the first half -------
  const float l = pair32(pair16(l_part, false), false);
  if (!row_ok) return;
  const int64_t stat_row = (int64_t)b * p.rows + n;
  const float m_nat = m_run == -INFINITY ? -INFINITY : m_run * p.scale;
  const int d0 = 256 * HALF + 4 * g4;
  if (direct) {
    const float inv = l > 0.f ? p.o_scale / l : 0.f;
    uint8_t* orow = p.o + (int64_t)qtok * p.o_tok + (int64_t)qhead * p.o_head;
    for (int j = 0; j < 2; ++j)
      for (int mt = 0; mt < 8; ++mt) {
        bf16x4 out;
        for (int i = 0; i < 4; ++i) out[i] = (__bf16)(oacc[j][mt][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 2 * (d0 + 128 * j + 16 * mt)) = out;
      }
    if (HALF == 0 && g4 == 0) p.lse[stat_row] = l > 0.f ? m_nat + logf(l) : -INFINITY;
  } else {
    const int64_t prow = (int64_t)slot * p.num_seqs * p.rows + stat_row;
    float* dst = p.ws_o + prow * kDv + d0;
    for (int j = 0; j < 2; ++j)
      for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(dst + 128 * j + 16 * mt) = oacc[j][mt];
    if (HALF == 0 && g4 == 0) p.ws_ml[prow] = float2{m_nat, l};
  }
}

// Grid (work items or bins, q-row tiles of 16 * groups rows); block 128 *
// groups threads; the half is a template parameter of the item, chosen once
// per wave.
template <bool CAUSAL_TAIL>
__global__ __launch_bounds__(128 * kPairMaxGroups) __attribute__((amdgpu_waves_per_eu(2)))
void mla_pair_kernel(MlaParams p, int groups) {
  extern __shared__ __attribute__((aligned(16))) uint8_t mla_pair_lds[];
  int it = blockIdx.x, it_end = blockIdx.x + 1;
  if (p.bin_offsets) {
    it = p.bin_offsets[blockIdx.x];
    it_end = p.bin_offsets[blockIdx.x + 1];
  }
  const bool odd = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1;
  const int it0 = it;
  for (; it < it_end; ++it) {
    if (odd)
      mla_pair_item<CAUSAL_TAIL, 1>(p, it, blockIdx.y, groups, mla_pair_lds, it == it0);
    else
      mla_pair_item<CAUSAL_TAIL, 0>(p, it, blockIdx.y, groups, mla_pair_lds, it == it0);
    __syncthreads();  // the next item's query overwrites LDS
  }
}

// ---- sparse slot-list form ------------------------------------------------------
// The decode of "vLLM PR #62633" (Kernel design) on these records: every
// decode token lists the slots it attends to (a sliding-window list and a
// top-k list, each over its own record pool); one workgroup per (tile of a
// list, 16 or 32 heads, token) runs the pair form over the tile's slots and
// writes a partial; the merge below combines a token's partials with the
// attention sink. Differences from the pair form:
//  * a key's record address comes from its list entry (a slot = page *
//    page_size + row): lane r16 of each 16-key block loads entry kb + r16
//    (a vector load, kPageAhead fetches ahead, as the pair form's page
//    entries), so every load has a per-lane 64-bit address;
//  * absent keys (a negative entry, one past the pool, or past the tile) read
//    slot 0 and are zeroed after the load (codes and scales, so no NaN from a
//    poisoned slot reaches PV) and masked to -inf;
//  * P * scale is split into a bf16 hi part and the bf16 rounding of the rest
//    (lo), and PV runs on both, so P enters the product with ~16 bits;
//  * no causal limit (every head sees every listed key) and always partials.
// Slots per tile of each list: one round of the ring (4 blocks of 16 keys).
// The page cuts the top-k list into 128-slot tiles (its MMA's M); here both
// lists use 64, twice the workgroups for a small step and half the chain of
// dependent loads per workgroup.
constexpr int kSparseTile0 = 64;  // sliding-window list
constexpr int kSparseTile1 = 64;  // top-k list

struct SparseList {
  const uint8_t* lat;
  int64_t lat_page, lat_row;  // bytes
  const uint8_t* rope;
  int64_t rope_page, rope_row;  // bytes
  const uint8_t* scl;
  int64_t scl_page, scl_row;  // bytes
  const int32_t* slots;
  int64_t slots_row;  // elements
  int width, page_shift, num_slots;
};

struct SparseParams {
  const uint8_t* q;
  int64_t q_tok, q_head;  // bytes
  SparseList list[2];
  const float* sink;
  uint8_t* o;
  int64_t o_tok, o_head;  // bytes
  float* lse;
  float* ws_o;    // [tiles][num_tokens][h_q][512]
  float2* ws_ml;  // [tiles][num_tokens][h_q]: (max in natural-log units, sum)
  float scale_log2e, scale, o_scale;
  int num_tokens, h_q, tiles0, tiles;
};

template <int HALF>
__device__ __forceinline__ void sparse_pair_item(const SparseParams& p, int tile, int rtile, int t, int groups,
                                                 uint8_t* lds) {
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int grp = w >> 1;

  const bool second = tile >= p.tiles0;
  const SparseList& L = second ? p.list[1] : p.list[0];
  const int j_begin = second ? (tile - p.tiles0) * kSparseTile1 : tile * kSparseTile0;
  const int j_end = min(j_begin + (second ? kSparseTile1 : kSparseTile0), L.width);
  const int32_t* list = L.slots + (int64_t)t * L.slots_row;
  const int pmask = (1 << L.page_shift) - 1;

  constexpr int kPageAhead = kPairStages - 1;
  // list entry of this lane's key in block kb (lanes of one key load the same entry)
  auto entry = [&](int kb) -> int { return list[min(kb + r16, j_end - 1)]; };
  int sv_ring[kPairStages];
  for (int u = 0; u < kPageAhead; ++u) sv_ring[u] = entry(j_begin + kBlockKeys * u);

  const int n = (rtile * groups + grp) * 16 + r16;  // query head; h_q is a multiple of 16
  bf16x8 qreg[kPairQSteps];
  {
    const uint8_t* qrow = p.q + (int64_t)t * p.q_tok + (int64_t)n * p.q_head;
    for (int k = 0; k < kPairQSteps; ++k) {
      const int blk = 2 * HALF + (k >> 2), s = k & 3;
      const int d = k < 8 ? 128 * blk + 64 * (s >> 1) + 16 * g4 + 8 * (s & 1) : kLatent + 32 * HALF + 8 * g4;
      qreg[k] = *reinterpret_cast<const bf16x8*>(qrow + 2 * d);
    }
  }
  const float c2 = p.scale_log2e;

  uint8_t* const wl = lds + w * kPairWaveBytes;
  uint8_t* const xl = lds + (w ^ 1) * kPairWaveBytes + kPairX;
  bf16x8(*qw)[64] = reinterpret_cast<bf16x8(*)[64]>(wl);
  for (int k = 0; k < kPairQSteps; ++k) qw[k][lane] = qreg[k];

  f32x4 oacc[2][8];
  for (int j = 0; j < 2; ++j)
    for (int mt = 0; mt < 8; ++mt) oacc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  if (j_end > j_begin) {
    struct Fetched {
      HalfRec r;
      bool ok;
    };
    auto load_block = [&](int kb, int sv) {
      Fetched f;
      f.ok = kb + r16 < j_end && sv >= 0 && sv < L.num_slots;
      const int s = f.ok ? sv : 0;
      const int64_t pg = s >> L.page_shift;
      const int row = s & pmask;
      const uint8_t* lr = L.lat + pg * L.lat_page + (int64_t)row * L.lat_row + 256 * HALF;
      for (int j = 0; j < 2; ++j)
        for (int h = 0; h < 2; ++h) f.r.kl[j][h] = *reinterpret_cast<const uint4*>(lr + 128 * j + 64 * h + 16 * g4);
      f.r.kr = *reinterpret_cast<const uint4*>(L.rope + pg * L.rope_page + (int64_t)row * L.rope_row +
                                               2 * (32 * HALF + 8 * g4));
      f.r.sc = *reinterpret_cast<const float2*>(L.scl + pg * L.scl_page + (int64_t)row * L.scl_row + 8 * HALF);
      return f;
    };
    auto fetch = [&](Fetched& f, int kb, const int s) {
      f = load_block(kb, sv_ring[s]);
      sv_ring[(s + kPageAhead) % kPairStages] = entry(kb + kPageAhead * kBlockKeys);
    };

    const int tr_base = hrow_base(4 * g4 + (r16 >> 2), 8 * (r16 & 3));
    auto process = [&](const Fetched& cur, int kb, const int xs) {
      asm volatile("" ::: "memory");
      // keys 4 g4 + i of this block that exist (ballot of the lanes r16 = key, g4 = 0)
      const uint64_t okm = __builtin_amdgcn_ballot_w64(cur.ok);
      HalfRec r = cur.r;
      if (!cur.ok) {  // a select on loaded values: no conditional load
        for (int j = 0; j < 2; ++j)
          for (int h = 0; h < 2; ++h) r.kl[j][h] = uint4{0u, 0u, 0u, 0u};
        r.kr = uint4{0u, 0u, 0u, 0u};
        r.sc = float2{0.f, 0.f};
      }
      *reinterpret_cast<float2*>(wl + kPairScl + 8 * r16) = r.sc;
      f32x4 acc[2];
      for (int j = 0; j < 2; ++j) {
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < 4; ++s) {
          const bf16x8 a = e4m3x8_to_bf16(half_of(r.kl[j][s >> 1], s & 1));
          *reinterpret_cast<bf16x8*>(wl + kPairV + hrow_base(r16, 32 * g4 + 16 * (s & 1)) + 256 * j +
                                     128 * (s >> 1)) = a;
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qw[4 * j + s][lane], acc[j], 0, 0, 0);
        }
      }
      const f32x4 accr =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.kr), qw[8][lane], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      asm volatile("" ::: "memory");
      float2 scl[4];
      for (int i = 0; i < 4; ++i) scl[i] = *reinterpret_cast<const float2*>(wl + kPairScl + 8 * (4 * g4 + i));
      f32x4 part;
      for (int i = 0; i < 4; ++i) part[i] = accr[i] + scl[i].x * acc[0][i] + scl[i].y * acc[1][i];
      *reinterpret_cast<f32x4*>(wl + kPairX + xs * 1024 + 16 * lane) = part;
      __syncthreads();
      const f32x4 other = *reinterpret_cast<const f32x4*>(xl + xs * 1024 + 16 * lane);
      float sv[4];
      for (int i = 0; i < 4; ++i) sv[i] = ((okm >> (4 * g4 + i)) & 1) ? part[i] + other[i] : -INFINITY;
      // ---- online softmax (the reference max may lag, as in the pair form) ----
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = pair32(pair16(mx, true), true);
      const float m_max = fmaxf(m_run, mx);
      const bool move = m_run == -INFINITY ? m_max != -INFINITY : (m_max - m_run) * c2 > kLazyLog2;
      const float m_new = move ? m_max : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float corr = __builtin_amdgcn_exp2f((m_run - m_use) * c2);
      float pr[4], psum = 0.f;
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f((sv[i] - m_use) * c2);
        psum += pr[i];
      }
      l_part = l_part * corr + psum;
      if (__builtin_amdgcn_ballot_w64(move)) {
        for (int j = 0; j < 2; ++j)
          for (int mt = 0; mt < 8; ++mt) oacc[j][mt] *= corr;
      }
      m_run = m_new;
      // ---- O^T += V^T (P * scale)^T, P * scale = hi + lo in bf16 -----------------
      for (int j = 0; j < 2; ++j) {
        bf16x4 ph, pl;
        for (int i = 0; i < 4; ++i) {
          const float v = pr[i] * (j ? scl[i].y : scl[i].x);
          ph[i] = (__bf16)v;
          pl[i] = (__bf16)(v - (float)ph[i]);
        }
        bf16x4 a[8];
        for (int mt = 0; mt < 8; ++mt) {
          const s16x4 t4 = lds_read_tr16(wl + kPairV + tr_base + 256 * j + 32 * mt);
          __builtin_memcpy(&a[mt], &t4, 8);
        }
        for (int mt = 0; mt < 8; ++mt)
          oacc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[mt], ph, oacc[j][mt], 0, 0, 0);
        for (int mt = 0; mt < 8; ++mt)
          oacc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a[mt], pl, oacc[j][mt], 0, 0, 0);
      }
    };

    Fetched ring[kPairStages];
#pragma unroll
    for (int s = 0; s < kPairStages - 1; ++s) {
      fetch(ring[s], j_begin + kBlockKeys * s, s);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    const int rounds = (j_end - j_begin + kBlockKeys * kPairStages - 1) / (kBlockKeys * kPairStages);
    for (int r = 0; r < rounds; ++r) {
      const int kb0 = j_begin + r * kBlockKeys * kPairStages;
#pragma unroll
      for (int s = 0; s < kPairStages; ++s) {
        const int kb = kb0 + kBlockKeys * s;
        fetch(ring[(s + kPairStages - 1) % kPairStages], kb + kBlockKeys * (kPairStages - 1),
              (s + kPairStages - 1) % kPairStages);
        process(ring[s], kb, s & 1);
      }
    }
  }

  // ---- epilogue: the tile's partial (this wave's d_v half) -------------------------
  const float l = pair32(pair16(l_part, false), false);
  const int64_t prow = ((int64_t)tile * p.num_tokens + t) * p.h_q + n;
  const float m_nat = m_run == -INFINITY ? -INFINITY : m_run * p.scale;
  float* dst = p.ws_o + prow * kDv + 256 * HALF + 4 * g4;
  for (int j = 0; j < 2; ++j)
    for (int mt = 0; mt < 8; ++mt) *reinterpret_cast<f32x4*>(dst + 128 * j + 16 * mt) = oacc[j][mt];
  if (HALF == 0 && g4 == 0) p.ws_ml[prow] = float2{m_nat, l};
}

// Grid (tiles, head tiles of 16 * groups heads, tokens); block 128 * groups.
__global__ __launch_bounds__(128 * kPairMaxGroups) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_pair_kernel(SparseParams p, int groups) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sparse_pair_lds[];
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1)
    sparse_pair_item<1>(p, blockIdx.x, blockIdx.y, blockIdx.z, groups, sparse_pair_lds);
  else
    sparse_pair_item<0>(p, blockIdx.x, blockIdx.y, blockIdx.z, groups, sparse_pair_lds);
}

// Combine of a token's tile partials, in tile order (list 0, then list 1),
// with the sink as one more term of the denominator (the LSE merge of the
// split-KV path plus a partial with O = 0, max = sink, sum = 1). One thread
// per (token, head, 4 d_v).
__global__ __launch_bounds__(256) void sparse_merge_kernel(SparseParams p) {
  constexpr int kRound = 16;  // partials whose (max, sum) and rows are loaded together
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)p.num_tokens * p.h_q;
  if (id >= rows * (kDv / 4)) return;
  const int64_t row = id / (kDv / 4);  // t * h_q + h
  const int d = (int)(id - row * (kDv / 4)) * 4;
  const int h = (int)(row % p.h_q);
  const int t = (int)(row / p.h_q);
  const float sink = p.sink ? p.sink[h] : -INFINITY;
  // the running maximum m_star may rise from round to round: sums and rows
  // gathered so far are rescaled to it (one exp per round)
  float m_star = sink, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < p.tiles; i0 += kRound) {
    float2 ml[kRound];
    f32x4 oj[kRound];
    for (int k = 0; k < kRound; ++k) {
      const int i = min(i0 + k, p.tiles - 1);
      ml[k] = p.ws_ml[(int64_t)i * rows + row];
      oj[k] = *reinterpret_cast<const f32x4*>(p.ws_o + ((int64_t)i * rows + row) * kDv + d);
    }
    float m_round = m_star;
    for (int k = 0; k < kRound; ++k)
      if (i0 + k < p.tiles && ml[k].y > 0.f) m_round = fmaxf(m_round, ml[k].x);
    if (m_round > m_star && m_star != -INFINITY) {
      const float c = expf(m_star - m_round);
      den *= c;
      num *= c;
    }
    m_star = m_round;
    for (int k = 0; k < kRound; ++k) {
      if (i0 + k >= p.tiles || !(ml[k].y > 0.f)) continue;
      const float wgt = expf(ml[k].x - m_star);
      den += wgt * ml[k].y;
      num += wgt * oj[k];
    }
  }
  if (p.sink) den += expf(sink - m_star);
  const float inv = den > 0.f ? p.o_scale / den : 0.f;
  bf16x4 out;
  for (int e = 0; e < 4; ++e) out[e] = (__bf16)(num[e] * inv);
  *reinterpret_cast<bf16x4*>(p.o + (int64_t)t * p.o_tok + (int64_t)h * p.o_head + 2 * d) = out;
  if (d == 0) p.lse[row] = den > 0.f ? m_star + logf(den) : -INFINITY;
}

// rows >= 64: the staged form; fewer rows: the pair form
bool staged(const pkv_decode_args& a) { return a.q_len * a.h_q >= kLdsRows; }

int pair_groups(const pkv_decode_args& a) {
  const int g = (a.q_len * a.h_q + 15) / 16;
  return g < kPairMaxGroups ? g : kPairMaxGroups;
}

const void* select_kernel(const pkv_decode_args& a) {
  const bool ct = a.causal && a.q_len > 1;
  if (staged(a))
    return ct ? reinterpret_cast<const void*>(&mla_lds_kernel<true>)
              : reinterpret_cast<const void*>(&mla_lds_kernel<false>);
  return ct ? reinterpret_cast<const void*>(&mla_pair_kernel<true>)
            : reinterpret_cast<const void*>(&mla_pair_kernel<false>);
}

int waves_per_wg(const pkv_decode_args& a) { return staged(a) ? kLdsWaves : 2 * pair_groups(a); }

size_t dyn_lds_bytes(const pkv_decode_args& a) {
  if (staged(a)) return (size_t)kLdsBytes;
  return (size_t)2 * pair_groups(a) * kPairWaveBytes;
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

const char* mla_kernel_name(const pkv_decode_args& a) { return staged(a) ? "mla_lds_kernel" : "mla_pair_kernel"; }

int mla_rows_per_tile(const pkv_decode_args& a) { return staged(a) ? kLdsRows : 16 * pair_groups(a); }

hipError_t mla_occupancy(const pkv_decode_args& a, int* units_per_cu) {
  // one unit = one workgroup (all rows of one q-row tile of a work item)
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(units_per_cu, select_kernel(a),
                                                                    64 * waves_per_wg(a), dyn_lds_bytes(a));
  // the pair form with one row group fits four workgroups per CU, but the
  // plan is sized for three: a one-wave plan for four left some CUs with four
  // items and others with three, and the CUs with four set the end
  // (measured on the latent workload at one query token, same box: decode
  // 62.8 -> 60.7 us, merge 11.4 -> 9.6 us, step 75.2 -> 72.2 us; two per CU:
  // 64.8 us)
  if (e == hipSuccess && !staged(a) && pair_groups(a) == 1 && *units_per_cu > 3) *units_per_cu = 3;
  return e;
}

hipError_t mla_launch(const pkv_decode_args& a, hipStream_t stream) {
  MlaParams p;
  p.q = static_cast<const uint8_t*>(a.q);
  p.q_tok = a.q_tok_stride * 2;
  p.q_head = a.q_head_stride * 2;
  p.lat = a.k;
  p.lat_page = a.k_page_stride;
  p.lat_row = a.k_row_stride;
  p.rope = reinterpret_cast<const uint8_t*>(a.k_rope);
  p.rope_page = a.rope_page_stride * 2;
  p.rope_row = a.rope_row_stride * 2;
  p.scl = reinterpret_cast<const uint8_t*>(a.k_blk_scale);
  p.scl_page = a.scale_page_stride * 4;
  p.scl_row = a.scale_row_stride * 4;
  p.block_table = a.block_table;
  p.bt_row = a.bt_row_stride;
  p.seq_lens = a.seq_lens;
  p.o = static_cast<uint8_t*>(a.o);
  p.o_tok = a.o_tok_stride * 2;
  p.o_head = a.o_head_stride * 2;
  p.lse = a.lse;
  p.work = reinterpret_cast<const int4*>(a.work);
  p.n_splits = a.n_splits;
  const int64_t rows_all = ws_rows(a);
  p.ws_o = static_cast<float*>(a.workspace);
  p.ws_ml = a.workspace ? reinterpret_cast<float2*>(p.ws_o + (int64_t)a.max_splits * rows_all * kDv) : nullptr;
  p.bin_offsets = a.bin_offsets;
  p.scale_log2e = (float)((double)a.softmax_scale * 1.4426950408889634);
  p.scale = a.softmax_scale;
  p.o_scale = a.o_scale;
  p.num_seqs = a.num_seqs;
  p.q_len = a.q_len;
  p.h_q = a.h_q;
  p.rows = a.q_len * a.h_q;
  p.page_shift = log2_exact(a.page_size);
  p.num_pages = a.num_pages;
  p.max_blocks = a.max_blocks;
  p.max_splits = a.max_splits;
  const int wpw = waves_per_wg(a);
  int tiles = (p.rows + mla_rows_per_tile(a) - 1) / mla_rows_per_tile(a);
  int units = a.bin_offsets ? a.num_bins : a.num_work;
  const void* kernel = select_kernel(a);
  if (const hipError_t e = check_lds(kernel, dyn_lds_bytes(a)); e != hipSuccess) return e;
  if (staged(a)) {
    void* args[] = {&p, &units, &tiles};
    return hipLaunchKernel(kernel, dim3((unsigned)(units * tiles)), dim3(64 * wpw), args, dyn_lds_bytes(a), stream);
  }
  int groups = pair_groups(a);
  void* args[] = {&p, &groups};
  return hipLaunchKernel(kernel, dim3((unsigned)units, (unsigned)tiles), dim3(64 * wpw), args, dyn_lds_bytes(a),
                         stream);
}

int sparse_tiles(const pkv_sparse_args& a) {
  return (a.list[0].width + kSparseTile0 - 1) / kSparseTile0 + (a.list[1].width + kSparseTile1 - 1) / kSparseTile1;
}

int64_t sparse_ws_bytes(const pkv_sparse_args& a) {
  return (int64_t)sparse_tiles(a) * a.num_tokens * a.h_q * (kDv + 2) * 4;
}

hipError_t sparse_launch(const pkv_sparse_args& a, hipStream_t stream, bool tiles_kernel, bool merge_kernel) {
  SparseParams p;
  p.q = reinterpret_cast<const uint8_t*>(a.q);
  p.q_tok = a.q_tok_stride * 2;
  p.q_head = a.q_head_stride * 2;
  for (int i = 0; i < 2; ++i) {
    const pkv_sparse_list& s = a.list[i];
    SparseList& d = p.list[i];
    d.lat = s.latent;
    d.lat_page = s.lat_page_stride;
    d.lat_row = s.lat_row_stride;
    d.rope = reinterpret_cast<const uint8_t*>(s.rope);
    d.rope_page = s.rope_page_stride * 2;
    d.rope_row = s.rope_row_stride * 2;
    d.scl = reinterpret_cast<const uint8_t*>(s.blk_scale);
    d.scl_page = s.scale_page_stride * 4;
    d.scl_row = s.scale_row_stride * 4;
    d.slots = s.slots;
    d.slots_row = s.slots_row_stride;
    d.width = s.width;
    d.page_shift = s.width > 0 ? log2_exact(s.page_size) : 0;
    d.num_slots = s.width > 0 ? s.num_pages * s.page_size : 0;
  }
  p.sink = a.sink;
  p.o = reinterpret_cast<uint8_t*>(a.o);
  p.o_tok = a.o_tok_stride * 2;
  p.o_head = a.o_head_stride * 2;
  p.lse = a.lse;
  const int tiles = sparse_tiles(a);
  const int64_t rows = (int64_t)a.num_tokens * a.h_q;
  p.ws_o = static_cast<float*>(a.workspace);
  p.ws_ml = reinterpret_cast<float2*>(p.ws_o + (int64_t)tiles * rows * kDv);
  p.scale_log2e = (float)((double)a.softmax_scale * 1.4426950408889634);
  p.scale = a.softmax_scale;
  p.o_scale = a.o_scale;
  p.num_tokens = a.num_tokens;
  p.h_q = a.h_q;
  p.tiles0 = (a.list[0].width + kSparseTile0 - 1) / kSparseTile0;
  p.tiles = tiles;
  if (tiles > 0 && tiles_kernel) {
    int groups = a.h_q % 32 == 0 ? 2 : 1;
    void* args[] = {&p, &groups};
    const void* kernel = reinterpret_cast<const void*>(&sparse_pair_kernel);
    const size_t lds = (size_t)2 * groups * kPairWaveBytes;
    if (const hipError_t e = check_lds(kernel, lds); e != hipSuccess) return e;
    const hipError_t e = hipLaunchKernel(kernel,
                                         dim3((unsigned)tiles, (unsigned)(a.h_q / (16 * groups)), (unsigned)a.num_tokens),
                                         dim3(128 * groups), args, lds, stream);
    if (e != hipSuccess) return e;
  }
  if (!merge_kernel) return hipSuccess;
  void* margs[] = {&p};
  const int64_t threads = rows * (kDv / 4);
  return hipLaunchKernel(reinterpret_cast<const void*>(&sparse_merge_kernel), dim3((unsigned)((threads + 255) / 256)),
                         dim3(256), margs, 0, stream);
}

// stamps of the staged loop (stamped builds; hipErrorNotSupported otherwise)
hipError_t mla_copy_stamps(void* host_dst) { return PKV_STAMP_COPY(host_dst); }

}  // namespace pkv
