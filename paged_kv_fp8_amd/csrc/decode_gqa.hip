// Split-KV paged decode attention over an e4m3 K/V cache, d = 128, for
// gfx950 (MI355X).
//
// Method: "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", module
// docstring (tensor contract, qi-major query packing, causal tail / block
// mode, split-KV work items, direct write of unsplit sequences) and its
// decode kernel (online softmax with the running max kept in raw-score
// units, the -inf guard, the sum of unrounded probabilities, descales folded
// into the exponent and the output scale, lazy rescale of O). The MMA
// orientation -- keys on the M side, the few query rows of a GQA group on N
// -- is the swap-AB idea of "vLLM PR #62633" (Kernel design, MMA shape).
//
// gfx950 design (not the pages'):
//  * One wavefront per kv head: a workgroup of 64 * HW threads holds the HW
//    kv heads of one (work item, q-row tile) (HW = the largest power of two
//    dividing h_k, at most 8; 4 with two 16-row blocks per wave), so its
//    waves read the same pages together. Each wave streams its chunk of keys
//    32 at a time straight from HBM into registers, a ring of blocks ahead of
//    the math; there is no LDS staging of K/V and no barrier.
//  * QK^T: v_mfma_f32_16x16x32_{bf16,fp8}, A = 16 keys x 32 head-dim slots,
//    B = the q rows. Because the head-dim contraction is order-free, a lane's
//    A slots are whatever 32 bytes of its key row it loaded with two 16-byte
//    loads (bytes 16*g4.. and 64+16*g4..); q is loaded once with the same
//    permutation.
//  * PV: O^T (d_v x rows) += V^T (d_v x 32 keys) * P^T (32 keys x rows). The
//    key order of the contraction is chosen equal to the order in which the
//    QK^T accumulator already holds P (lane (n, g4) holds keys 4*g4+i and
//    16+4*g4+i), so P needs no lane exchange. V^T is built in registers: a
//    lane loads 8 consecutive d_v bytes of each of its 8 keys (coalesced: 4
//    rows x 128 B per load instruction) and transposes them with v_perm_b32
//    (plus the exact e4m3 -> bf16 converts on the bf16 path). dv-tile mt row
//    m is d_v index 8*m + mt, which makes each lane's final O a run of 32
//    contiguous d_v values of one query row.
//  * Row statistics: the max needs two cross-lane steps (lanes 16 and 32
//    apart); the sum stays per lane until the epilogue.
//  * Page lookups: the two pages of a 32-key block (page_size >= 16, so a
//    16-key group never straddles pages) come from a small vector load
//    issued two blocks ahead and are read with readlane. Keys are clamped to the chunk's last key (a
//    real, finite row; masked), so no block-table entry at or past
//    ceil(L / page_size) and no cache row at or past L is ever read.
//  * Every main-loop step issues the same 13 loads whether or not its block
//    exists, so the wait before consuming a block covers that block only and
//    the ring of STAGES blocks stays in flight.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "pkv_internal.h"
#include "stamps.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;          // head dim (qk and v)
constexpr int kTileKeys = 128;   // planner tile
constexpr int kBlockKeys = 32;   // keys per main-loop step
constexpr float kP8Scale = 448.0f;  // fp8 P is stored as e4m3(p * 448)
constexpr float kLog2P8Scale = 8.807354922057604f;  // log2(448): p * 448 = exp2(... + log2 448)
constexpr float kLazyLog2 = 8.0f;   // bf16 P: reference max may lag until p would exceed 2^8

struct GqaParams {
  const uint8_t* q;   // byte address
  int64_t q_tok, q_head;  // bytes
  const uint8_t* k;
  int64_t k_page, k_row, k_head;  // bytes
  const uint8_t* v;
  int64_t v_page, v_row, v_head;
  const int32_t* block_table;
  int64_t bt_row;
  const int32_t* seq_lens;
  const float* qd;
  int64_t qd_seq, qd_head;
  const float* kd;
  int64_t kd_seq, kd_head;
  const float* vd;
  int64_t vd_seq, vd_head;
  uint8_t* o;
  int64_t o_tok, o_head;  // bytes
  float* lse;
  const int4* work;
  const int32_t* n_splits;
  float* ws_o;   // [max_splits][num_seqs][h_k][rows][128]
  float2* ws_ml; // [max_splits][num_seqs][h_k][rows]
  const int32_t* bin_offsets;  // [bins + 1] or null: one work item per workgroup
  int32_t* queue;              // [2][h_k * q tiles] or null: no shared queue (persistent form)
  float scale_log2e, scale, o_scale;
  int num_seqs, q_len, h_k, h_r, rows, page_shift, num_pages, max_blocks, max_splits;
  int key_mult;  // keys per unit of a work item's range: 128 (tile plans) or 1 (key plans)
  int num_work;
  int q_tiles;    // q-row tiles per work item
  int xcd_tiles;  // one-item form with q_tiles > 1: blockIdx.x enumerates (item, tile), tiles of an item on one XCD
  const uint8_t* ks;  // NVFP4: e4m3 group scales of K and V (one byte per 16 values)
  int64_t ks_page, ks_row, ks_head;  // bytes
  const uint8_t* vs;
  int64_t vs_page, vs_row, vs_head;
  int paired;  // work in pairs: workgroup x runs items 2x, 2x + 1 (eight waves, four kv heads)
};

__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint2 x) {
  // exact: every e4m3 value is a bf16 value
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.x, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x.y, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ uint2 half_of(uint4 x, int h) { return h ? uint2{x.z, x.w} : uint2{x.x, x.y}; }

__device__ __forceinline__ long as_long(uint2 x) {
  return (long)(((unsigned long long)x.y << 32) | x.x);
}

// Butterfly steps across the four lanes {l, l^16, l^32, l^48} that hold one
// query row. v_permlane{16,32}_swap with both operands = x return the pair
// {x[l], x[l^16]} (resp. l^32) in an order that is the same on both partner
// lanes, so max/sum of the pair is bit-identical on the two lanes. Plain VALU
// ops: no LDS permute, so no lgkmcnt wait that would also wait for the
// scalar page loads.
__device__ __forceinline__ float pair16(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float pair32(float x, bool take_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return take_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float wave_max16(float x) { return pair32(pair16(x, true), true); }
__device__ __forceinline__ float wave_sum16(float x) { return pair32(pair16(x, false), false); }

// Raw bytes of one 32-key block as this lane loads them.
struct RawBlock {
  uint4 k[2][2];  // [M tile t][half]: key kb+16t+r16, bytes 16*g4.. and 64+16*g4..
  uint2 v[8];     // key kb+16*(j>>2)+4*g4+(j&3), bytes 8*r16 .. 8*r16+7
};

// B operand of QK^T: lane (n = r16, g4), k-step s holds
// q[n][64*(s>>1) + 16*g4 + 8*(s&1) + 0..7] (bf16 rows, or e4m3 codes).
template <int NB>
struct QOperand {
  bf16x8 qb[NB][4];
  long q8[NB][4];
};

// Running softmax state of a wave's query rows: lane (r16, g4) holds
// O^T[d_v = 32*g4 + 8*i + mt][row r16] in oacc[nb][mt][i], the row's running
// max (raw-score units) and its lane-partial sum of probabilities.
template <int NB>
struct RowState {
  f32x4 oacc[NB][8];
  float m_run[NB], l_part[NB];
};

template <int NB>
__device__ __forceinline__ void reset_rows(RowState<NB>& st) {
  for (int nb = 0; nb < NB; ++nb) {
    for (int mt = 0; mt < 8; ++mt) st.oacc[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_run[nb] = -INFINITY;
    st.l_part[nb] = 0.f;
  }
}

// Query rows of this wave: packed row n = row0 + 16*nb + r16 is query token
// qi = n / h_r of sequence b, query head g*h_r + n % h_r.
template <int NB>
struct RowMap {
  bool ok[NB];
  int qi[NB], hr[NB];
};

template <int NB>
__device__ __forceinline__ RowMap<NB> row_map(const GqaParams& p, int row0, int r16) {
  RowMap<NB> m;
  for (int nb = 0; nb < NB; ++nb) {
    const int n = row0 + 16 * nb + r16;
    m.ok[nb] = n < p.rows;
    m.qi[nb] = n / p.h_r;
    m.hr[nb] = n - m.qi[nb] * p.h_r;
  }
  return m;
}

template <bool FP8Q, int NB>
__device__ __forceinline__ void load_q(const GqaParams& p, QOperand<NB>& q, const RowMap<NB>& rm, int b, int g,
                                       int g4) {
  for (int nb = 0; nb < NB; ++nb) {
    const uint8_t* qrow =
        p.q + (int64_t)(b * p.q_len + rm.qi[nb]) * p.q_tok + (int64_t)(g * p.h_r + rm.hr[nb]) * p.q_head;
    for (int s = 0; s < 4; ++s) {
      const int d = 64 * (s >> 1) + 16 * g4 + 8 * (s & 1);
      if (FP8Q) {
        q.q8[nb][s] = rm.ok[nb] ? *reinterpret_cast<const long*>(qrow + d) : 0;
      } else {
        if (rm.ok[nb]) {
          q.qb[nb][s] = *reinterpret_cast<const bf16x8*>(qrow + 2 * d);
        } else {
          for (int e = 0; e < 8; ++e) q.qb[nb][s][e] = (__bf16)0.0f;
        }
      }
    }
  }
}

// Lane-constant parts of the KV load offsets inside a 16-key group of a page
// (row r16 / rows 4*g4 + i of the group), and of the clamp bound added to
// a group's last-row offset.
struct LaneOffsets {
  uint32_t k, kb;     // K: r16 * k_row + 16 g4; 16 g4
  uint32_t v[4], vb;  // V: (4 g4 + i) * v_row + 8 r16; 8 r16
};

__device__ __forceinline__ LaneOffsets lane_offsets(const GqaParams& p, int r16, int g4) {
  LaneOffsets o;
  o.k = (uint32_t)r16 * (uint32_t)p.k_row + 16u * (uint32_t)g4;
  o.kb = 16u * (uint32_t)g4;
  for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)(4 * g4 + i) * (uint32_t)p.v_row + 8u * (uint32_t)r16;
  o.vb = 8u * (uint32_t)r16;
  return o;
}

// Byte offset of page pg in a pool: pg is clamped into [0, num_pages) (so
// below 2^31) and every page stride is below 2^32 bytes (checked on the
// host), so one 32 x 32 -> 64-bit product suffices (two scalar multiplies,
// where a 64-bit product of the signed index takes four and a sign extension).
__device__ __forceinline__ uint64_t page_off(int64_t pg, int64_t page_stride) {
  return (uint64_t)(uint32_t)pg * (uint64_t)(uint32_t)page_stride;
}

// The 13 loads of one 32-key block (keys kb.. clamped to last_key) of kv
// head g from the two pages pg0 (keys kb..kb+15) and pg1 (kb+16..kb+31).
// Group t starts at key s_t = min(kb + 16 t, last_key), row s_t & pmask of
// its page (a 16-key group never straddles pages); that part of the address
// is wave-uniform and goes into the scalar base of each load. A lane's row
// inside the group is clamped to last_key - s_t, done on byte offsets
// (min(row, lim) * stride = min(row * stride, lim * stride)), so a block
// costs one add per group and one min per load of per-lane arithmetic.
__device__ __forceinline__ RawBlock load_block(const GqaParams& p, int g, int kb, int pg0, int pg1, int last_key,
                                               int pmask, const LaneOffsets& lo) {
  RawBlock r;
  for (int t = 0; t < 2; ++t) {
    const int st = min(kb + 16 * t, last_key);
    const uint32_t lim = (uint32_t)max(last_key - st, 0);
    const int64_t pg = t ? pg1 : pg0;
    const uint32_t row = (uint32_t)(st & pmask);
    const uint8_t* kbase = p.k + page_off(pg, p.k_page) + (int64_t)g * p.k_head + row * (uint32_t)p.k_row;
    const uint8_t* vbase = p.v + page_off(pg, p.v_page) + (int64_t)g * p.v_head + row * (uint32_t)p.v_row;
    const uint32_t koff = min(lo.k, lim * (uint32_t)p.k_row + lo.kb);
    r.k[t][0] = *reinterpret_cast<const uint4*>(kbase + koff);
    r.k[t][1] = *reinterpret_cast<const uint4*>(kbase + (koff + 64u));
    const uint32_t vlim = lim * (uint32_t)p.v_row + lo.vb;
    for (int i = 0; i < 4; ++i) r.v[4 * t + i] = *reinterpret_cast<const uint2*>(vbase + min(lo.v[i], vlim));
  }
  return r;
}

// ---- packed fp4 (e2m1) K/V --------------------------------------------------
// A cache row holds d = 128 codes in 64 bytes, element 2i in the low nibble
// of byte i ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", narrow KV
// formats and pack_subbyte).
//
// Raw bytes of one 32-key block as this lane loads them: K for the QK^T
// operand of v_mfma_scale_f32_16x16x128_f8f6f4 (the 32 codes d = 32*g4 ..
// 32*g4+31 of key kb+16t+r16, one 16-byte run), V as 8 codes (d_v 8*r16 ..)
// of each of the lane's 8 keys. With an fp4 A and an e4m3 B operand the
// instruction pairs the A nibbles of lane group g with the B bytes of lane
// groups {0, 2} (g even) or {1, 3} (g odd) in 16-element chunks; measured
// slot by slot, that puts d = 32*g4.. here against exactly the head dims the
// e4m3 query operand (d = 64*(s>>1) + 16*g4 + 8*(s&1) ..) holds.
struct RawBlock4 {
  uint4 k[2];
  uint32_t v[8];
};

struct LaneOffsets4 {
  uint32_t k, kb;     // K: r16 * k_row + 16 g4; 16 g4
  uint32_t v[4], vb;  // V: (4 g4 + i) * v_row + 4 r16; 4 r16
};

__device__ __forceinline__ LaneOffsets4 lane_offsets4(const GqaParams& p, int r16, int g4) {
  LaneOffsets4 o;
  o.k = (uint32_t)r16 * (uint32_t)p.k_row + 16u * (uint32_t)g4;
  o.kb = 16u * (uint32_t)g4;
  for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)(4 * g4 + i) * (uint32_t)p.v_row + 4u * (uint32_t)r16;
  o.vb = 4u * (uint32_t)r16;
  return o;
}

// load_block for packed fp4 rows: 2 + 8 loads, same row clamping.
__device__ __forceinline__ RawBlock4 load_block4(const GqaParams& p, int g, int kb, int pg0, int pg1, int last_key,
                                                 int pmask, const LaneOffsets4& lo) {
  RawBlock4 r;
  for (int t = 0; t < 2; ++t) {
    const int st = min(kb + 16 * t, last_key);
    const uint32_t lim = (uint32_t)max(last_key - st, 0);
    const int64_t pg = t ? pg1 : pg0;
    const uint32_t row = (uint32_t)(st & pmask);
    const uint8_t* kbase = p.k + page_off(pg, p.k_page) + (int64_t)g * p.k_head + row * (uint32_t)p.k_row;
    const uint8_t* vbase = p.v + page_off(pg, p.v_page) + (int64_t)g * p.v_head + row * (uint32_t)p.v_row;
    const uint32_t koff = min(lo.k, lim * (uint32_t)p.k_row + lo.kb);
    r.k[t] = *reinterpret_cast<const uint4*>(kbase + koff);
    const uint32_t vlim = lim * (uint32_t)p.v_row + lo.vb;
    for (int i = 0; i < 4; ++i) r.v[4 * t + i] = *reinterpret_cast<const uint32_t*>(vbase + min(lo.v[i], vlim));
  }
  return r;
}

// Eight e2m1 codes (element 2i in the low nibble of byte i) -> their e4m3
// bytes, exact (every e2m1 value is an e4m3 value), split by parity:
// .x = elements 0, 2, 4, 6 and .y = elements 1, 3, 5, 7. The magnitude (3
// bits) picks one of 8 bytes with v_perm_b32 (0, 0.5, 1, 1.5, 2, 3, 4, 6 as
// 0x00 0x30 0x38 0x3C 0x40 0x44 0x48 0x4C); the sign (bit 3 of the code) goes
// to bit 7, where a high nibble already has it.
__device__ __forceinline__ uint2 e2m1x8_to_e4m3(uint32_t x) {
  const uint32_t lo = __builtin_amdgcn_perm(0x4C484440u, 0x3C383000u, x & 0x07070707u);
  const uint32_t hi = __builtin_amdgcn_perm(0x4C484440u, 0x3C383000u, (x >> 4) & 0x07070707u);
  return uint2{lo | ((x << 4) & 0x80808080u), hi | (x & 0x80808080u)};
}

// Packed fp6 rows (e2m3 or e3m2, 96 bytes per row of 128 codes, element i at
// bits 6i .. 6i+5; "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", KV
// cache formats and pack_subbyte). The scaled MFMA reads an fp6 A operand as
// that same bitstream, 32 codes in 6 VGPRs, with the fp4 slot map (measured
// slot by slot), so lane group g4 takes the 24 bytes of head dims 32*g4 ..
// 32*g4+31. V: the 8 codes d_v 8*r16 .. of a key are 6 bytes at byte 6*r16;
// each lane loads the 8-byte window at 6*r16 rounded down to 4 bytes (its
// codes start 0 or 2 bytes in; the window never passes the row's end).
struct RawBlock6 {
  uint2 k[2][3];
  uint2 v[8];
};

struct LaneOffsets6 {
  uint32_t k, kb;     // K: r16 * k_row + 24 g4; 24 g4
  uint32_t v[4], vb;  // V: (4 g4 + i) * v_row + w; w = (6 r16) & ~3
  uint32_t sel[3];    // v_perm selectors gathering two keys' 12 code bytes from their windows
};

__device__ __forceinline__ LaneOffsets6 lane_offsets6(const GqaParams& p, int r16, int g4) {
  LaneOffsets6 o;
  o.k = (uint32_t)r16 * (uint32_t)p.k_row + 24u * (uint32_t)g4;
  o.kb = 24u * (uint32_t)g4;
  const uint32_t w = (6u * (uint32_t)r16) & ~3u;
  for (int i = 0; i < 4; ++i) o.v[i] = (uint32_t)(4 * g4 + i) * (uint32_t)p.v_row + w;
  o.vb = w;
  const bool odd = (6 * r16) & 2;  // codes start 2 bytes into the window
  o.sel[0] = odd ? 0x05040302u : 0x03020100u;  // key a bytes 0..3
  o.sel[1] = odd ? 0x07060302u : 0x05040100u;  // key a bytes 4, 5 | key b bytes 0, 1
  o.sel[2] = odd ? 0x07060504u : 0x05040302u;  // key b bytes 2..5
  return o;
}

typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2))) __attribute__((aligned(4)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef _Float16 f16x32 __attribute__((ext_vector_type(32)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// load_block for packed fp6 rows: 6 + 8 loads, same row clamping.
__device__ __forceinline__ RawBlock6 load_block6(const GqaParams& p, int g, int kb, int pg0, int pg1, int last_key,
                                                 int pmask, const LaneOffsets6& lo) {
  RawBlock6 r;
  for (int t = 0; t < 2; ++t) {
    const int st = min(kb + 16 * t, last_key);
    const uint32_t lim = (uint32_t)max(last_key - st, 0);
    const int64_t pg = t ? pg1 : pg0;
    const uint32_t row = (uint32_t)(st & pmask);
    const uint8_t* kbase = p.k + page_off(pg, p.k_page) + (int64_t)g * p.k_head + row * (uint32_t)p.k_row;
    const uint8_t* vbase = p.v + page_off(pg, p.v_page) + (int64_t)g * p.v_head + row * (uint32_t)p.v_row;
    const uint32_t koff = min(lo.k, lim * (uint32_t)p.k_row + lo.kb);
    for (int j = 0; j < 3; ++j) r.k[t][j] = *reinterpret_cast<const uint2*>(kbase + (koff + 8u * j));
    const uint32_t vlim = lim * (uint32_t)p.v_row + lo.vb;
    for (int i = 0; i < 4; ++i) {
      const u32x2_a4 x = *reinterpret_cast<const u32x2_a4*>(vbase + min(lo.v[i], vlim));
      r.v[4 * t + i] = uint2{x[0], x[1]};
    }
  }
  return r;
}

// Four keys' V codes (windows a0, a1, b0, b1) -> their e4m3 bytes: the 32
// codes are packed into one 192-bit bitstream, widened to f16 with
// v_cvt_scalef32_pk32_f16_{fp6,bf6} and narrowed to e4m3 two at a time; all
// three steps are exact (every e2m3 and e3m2 value is an e4m3 value).
template <int KVF>
__device__ __forceinline__ void fp6x32_to_e4m3(const uint2* win, const LaneOffsets6& lo, uint2* out) {
  i32x6 x;
  for (int pr = 0; pr < 2; ++pr) {
    const uint2 a = win[2 * pr], b = win[2 * pr + 1];
    x[3 * pr + 0] = (int)__builtin_amdgcn_perm(a.y, a.x, lo.sel[0]);
    x[3 * pr + 1] = (int)__builtin_amdgcn_perm(b.x, a.y, lo.sel[1]);
    x[3 * pr + 2] = (int)__builtin_amdgcn_perm(b.y, b.x, lo.sel[2]);
  }
  f16x32 h;
  if constexpr (KVF == PKV_KV_E2M3)
    h = __builtin_amdgcn_cvt_scalef32_pk32_f16_fp6(x, 1.0f);
  else
    h = __builtin_amdgcn_cvt_scalef32_pk32_f16_bf6(x, 1.0f);
  for (int i = 0; i < 4; ++i) {
    uint32_t w[2];
    for (int hw = 0; hw < 2; ++hw) {
      // the first conversion's other word is its own (dead) input: no zeroed register
      const f16x2 a = {h[8 * i + 4 * hw], h[8 * i + 4 * hw + 1]};
      s16x2 v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(__builtin_bit_cast(s16x2, a), a, 1.0f, false);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(v, f16x2{h[8 * i + 4 * hw + 2], h[8 * i + 4 * hw + 3]}, 1.0f, true);
      w[hw] = __builtin_bit_cast(uint32_t, v);
    }
    out[i] = uint2{w[0], w[1]};
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One 32-key block: S = K Q^T, online softmax, O^T += V^T P^T. lim[nb] is
// the last key row r16 of block nb may see; keys past lim_min need the mask.
// Query operand parked in LDS (two row blocks: saves the registers that would
// otherwise push the O accumulators into AGPRs): entry (nb, s) of lane l at
// qlds + ((4 nb + s) * 64 + l) * size, one conflict-free read per k-step.
template <bool FP8Q, int NB>
__device__ __forceinline__ void park_q(const QOperand<NB>& q, uint8_t* qlds, int lane) {
  for (int nb = 0; nb < NB; ++nb)
    for (int s = 0; s < 4; ++s) {
      if (FP8Q)
        *reinterpret_cast<long*>(qlds + ((4 * nb + s) * 64 + lane) * 8) = q.q8[nb][s];
      else
        *reinterpret_cast<bf16x8*>(qlds + ((4 * nb + s) * 64 + lane) * 16) = q.qb[nb][s];
    }
}

// Online softmax of one 32-key block's scores and O^T += V^T P^T, with the
// block's V as e4m3 (fp8 path) codes or as the bytes the bf16 path converts
// exactly: vraw[j] holds key kb + 16 (j >> 2) + 4 g4 + (j & 3), d_v bytes
// 8 r16 .. 8 r16 + 7 of this lane.
// With V_BY_PARITY (converted fp4 codes) .x holds d_v bytes 8 r16 + 0, 2, 4,
// 6 and .y bytes 8 r16 + 1, 3, 5, 7, and the Oᵀ tiles are indexed to match.
template <bool FP8Q, int NB, bool V_BY_PARITY = false>
__device__ __forceinline__ void softmax_pv(f32x4 (&sacc)[NB][2], const uint2 (&vraw)[8], int kb, RowState<NB>& st,
                                           const int* lim, int lim_min, float c2, int g4) {
  // ---- online softmax (per query row = lane column r16) --------------------
  bf16x8 pb[NB];
  long p8[NB];
  const bool need_mask = kb + kBlockKeys - 1 > lim_min;
  for (int nb = 0; nb < NB; ++nb) {
    if (need_mask) {
      for (int t = 0; t < 2; ++t)
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * t + 4 * g4 + i > lim[nb]) sacc[nb][t][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[nb][0][0], sacc[nb][0][1]), fmaxf(sacc[nb][0][2], sacc[nb][0][3])),
                     fmaxf(fmaxf(sacc[nb][1][0], sacc[nb][1][1]), fmaxf(sacc[nb][1][2], sacc[nb][1][3])));
    mx = wave_max16(mx);
    // m_run is the row's reference max: P = exp2((s - m_run) * c2), with l
    // and O kept relative to it. e4m3 P (p * 448 must stay <= 448) moves it to
    // every new max. bf16 P moves it only once the new max would make some p
    // exceed 2^kLazyLog2 (or on the first visible key), so rows rarely need
    // the O rescale; the result is the same softmax, rounded in a different
    // place.
    const float m_max = fmaxf(st.m_run[nb], mx);
    const bool move = FP8Q ? m_max != st.m_run[nb]
                           : (st.m_run[nb] == -INFINITY ? m_max != -INFINITY
                                                        : (m_max - st.m_run[nb]) * c2 > kLazyLog2);
    const float m_new = move ? m_max : st.m_run[nb];
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: exp2(-inf) = 0
    const float corr = __builtin_amdgcn_exp2f((st.m_run[nb] - m_use) * c2);
    // one fma per score: exp2(s c2 - m c2), times 448 for e4m3 P (then l
    // sums p * 448 too, and the epilogue divides it out)
    const float off = (FP8Q ? kLog2P8Scale : 0.f) - m_use * c2;
    float pr[8];
    float psum = 0.f;
    for (int t = 0; t < 2; ++t)
      for (int i = 0; i < 4; ++i) {
        pr[4 * t + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nb][t][i], c2, off));
        psum += pr[4 * t + i];
      }
    st.l_part[nb] = st.l_part[nb] * corr + psum;
    // rescale O only if some row's reference moved (otherwise corr == 1 exactly)
    if (__builtin_amdgcn_ballot_w64(move)) {
      for (int mt = 0; mt < 8; ++mt) st.oacc[nb][mt] *= corr;
    }
    st.m_run[nb] = m_new;
    if (FP8Q) {
      // the first conversion of each word pair keeps its other word from a
      // dead input (overwritten by the second): no zeroed register
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(pr[0], pr[1], __float_as_int(pr[0]), false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(pr[2], pr[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(pr[4], pr[5], __float_as_int(pr[4]), false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(pr[6], pr[7], hi, true);
      p8[nb] = as_long(uint2{(unsigned)lo, (unsigned)hi});
    } else {
      for (int e = 0; e < 8; ++e) pb[nb][e] = (__bf16)pr[e];
    }
  }

  // ---- O^T += V^T P^T --------------------------------------------------------
  if (FP8Q) {
    // 4x4 byte transposes: quad kq of keys, word w of d_v bytes
    for (int w2 = 0; w2 < 2; ++w2) {
      unsigned col[2][4];  // [kq][e]: keys 4kq..4kq+3 at d_v 8*r16 + 4*w2 + e
      for (int kq = 0; kq < 2; ++kq) {
        const unsigned r0 = w2 ? vraw[4 * kq + 0].y : vraw[4 * kq + 0].x;
        const unsigned r1 = w2 ? vraw[4 * kq + 1].y : vraw[4 * kq + 1].x;
        const unsigned r2 = w2 ? vraw[4 * kq + 2].y : vraw[4 * kq + 2].x;
        const unsigned r3 = w2 ? vraw[4 * kq + 3].y : vraw[4 * kq + 3].x;
        const unsigned t0 = __builtin_amdgcn_perm(r0, r1, 0x01050004u);
        const unsigned t1 = __builtin_amdgcn_perm(r0, r1, 0x03070206u);
        const unsigned t2 = __builtin_amdgcn_perm(r2, r3, 0x01050004u);
        const unsigned t3 = __builtin_amdgcn_perm(r2, r3, 0x03070206u);
        col[kq][0] = __builtin_amdgcn_perm(t0, t2, 0x01000504u);
        col[kq][1] = __builtin_amdgcn_perm(t0, t2, 0x03020706u);
        col[kq][2] = __builtin_amdgcn_perm(t1, t3, 0x01000504u);
        col[kq][3] = __builtin_amdgcn_perm(t1, t3, 0x03020706u);
      }
      for (int e = 0; e < 4; ++e) {
        const long a = as_long(uint2{col[0][e], col[1][e]});
        const int mt = V_BY_PARITY ? 2 * e + w2 : 4 * w2 + e;
        for (int nb = 0; nb < NB; ++nb)
          st.oacc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, p8[nb], st.oacc[nb][mt], 0, 0, 0);
      }
    }
  } else {
    for (int w2 = 0; w2 < 2; ++w2) {
      unsigned xy[4][2];  // [key pair pp][0: d_v bytes 0,1 / 1: bytes 2,3 of the word], interleaved by key
      for (int pp = 0; pp < 4; ++pp) {
        const unsigned a0 = w2 ? vraw[2 * pp].y : vraw[2 * pp].x;
        const unsigned a1 = w2 ? vraw[2 * pp + 1].y : vraw[2 * pp + 1].x;
        xy[pp][0] = __builtin_amdgcn_perm(a0, a1, 0x01050004u);
        xy[pp][1] = __builtin_amdgcn_perm(a0, a1, 0x03070206u);
      }
      for (int e = 0; e < 4; ++e) {
        bf16x8 a;
        for (int pp = 0; pp < 4; ++pp) {
          const bf16x2 two = (e & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xy[pp][e >> 1], 1.0f, true)
                                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(xy[pp][e >> 1], 1.0f, false);
          a[2 * pp] = two[0];
          a[2 * pp + 1] = two[1];
        }
        const int mt = 4 * w2 + e;
        for (int nb = 0; nb < NB; ++nb)
          st.oacc[nb][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nb], st.oacc[nb][mt], 0, 0, 0);
      }
    }
  }
}

template <bool FP8Q, int NB, bool QLDS>
__device__ __forceinline__ void process_block(const RawBlock& cur, int kb, const QOperand<NB>& q, const uint8_t* qlds,
                                              RowState<NB>& st, const int* lim, int lim_min, float c2, int g4) {
  const int lane = threadIdx.x & 63;
  // keep the LDS query reads inside the loop (hoisted, they would occupy the
  // registers this form saves)
  if (QLDS) asm volatile("" ::: "memory");
  // ---- S = K Q^T (keys on M) -----------------------------------------------
  f32x4 sacc[NB][2];
  for (int nb = 0; nb < NB; ++nb)
    for (int t = 0; t < 2; ++t) sacc[nb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < 2; ++t) {
    for (int s = 0; s < 4; ++s) {
      const uint2 kraw = half_of(cur.k[t][s >> 1], s & 1);
      if (FP8Q) {
        const long a = as_long(kraw);
        for (int nb = 0; nb < NB; ++nb) {
          const long b = QLDS ? *reinterpret_cast<const long*>(qlds + ((4 * nb + s) * 64 + lane) * 8) : q.q8[nb][s];
          sacc[nb][t] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, sacc[nb][t], 0, 0, 0);
        }
      } else {
        const bf16x8 a = e4m3x8_to_bf16(kraw);
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 b =
              QLDS ? *reinterpret_cast<const bf16x8*>(qlds + ((4 * nb + s) * 64 + lane) * 16) : q.qb[nb][s];
          sacc[nb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sacc[nb][t], 0, 0, 0);
        }
      }
    }
  }
  softmax_pv<FP8Q, NB>(sacc, cur.v, kb, st, lim, lim_min, c2, g4);
}

// One 32-key block of packed fp4 K/V with an e4m3 query: S = K Q^T on
// v_mfma_scale_f32_16x16x128_f8f6f4 (A = 16 keys x 128 head-dim fp4 codes,
// B = the e4m3 query rows, block scales 1.0: one instruction per 16 keys),
// then V converted to e4m3 and the fp8 softmax / PV.
template <int NB, bool QLDS>
__device__ __forceinline__ void process_block_fp4(const RawBlock4& cur, int kb, const QOperand<NB>& q,
                                                  const uint8_t* qlds, RowState<NB>& st, const int* lim, int lim_min,
                                                  float c2, int g4) {
  const int lane = threadIdx.x & 63;
  if (QLDS) asm volatile("" ::: "memory");
  f32x4 sacc[NB][2];
  for (int t = 0; t < 2; ++t) {
    const i32x8 a = {(int)cur.k[t].x, (int)cur.k[t].y, (int)cur.k[t].z, (int)cur.k[t].w, 0, 0, 0, 0};
    for (int nb = 0; nb < NB; ++nb) {
      long qv[4];
      for (int s = 0; s < 4; ++s)
        qv[s] = QLDS ? *reinterpret_cast<const long*>(qlds + ((4 * nb + s) * 64 + lane) * 8) : q.q8[nb][s];
      const i32x8 b = {(int)qv[0], (int)(qv[0] >> 32), (int)qv[1], (int)(qv[1] >> 32),
                       (int)qv[2], (int)(qv[2] >> 32), (int)qv[3], (int)(qv[3] >> 32)};
      // A format 4 = fp4 e2m1, B format 0 = fp8 e4m3; E8M0 scales 127 = 2^0
      sacc[nb][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 4, 0, 0,
                                                                      127, 0, 127);
    }
  }
  uint2 v8[8];
  for (int j = 0; j < 8; ++j) v8[j] = e2m1x8_to_e4m3(cur.v[j]);
  softmax_pv<true, NB, true>(sacc, v8, kb, st, lim, lim_min, c2, g4);
}

// NVFP4 rows ("mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", KV cache
// formats and nvfp4_quantize): packed e2m1 codes as for fp4 plus one e4m3
// scale per 16 head-dim values. The decode multiplies the values
// e4m3(code * scale * 2^-3): the e4m3 scale is not a power of two, so the
// codes cannot go to the scaled MFMA (its block scales are E8M0 per 32) and
// the rounding is part of the method. Each block is converted to the e4m3
// block of the e4m3 cache and runs that path: a lane loads its e4m3 lane
// layout's head dims (K: 16*g4 .. and 64 + 16*g4 .., 8 bytes each, with the
// key's 8 group scales; V: 8 codes d_v 8*r16 .. of each of its 8 keys and
// their group scale byte r16 / 2).
struct RawBlockN {
  uint2 k[2][2];   // [t][half] packed codes
  uint2 ks[2];     // [t] the key's 8 group scales
  uint32_t v[8];   // packed codes
  uint32_t vs[8];  // group scale byte
};

struct LaneOffsetsN {
  uint32_t k, kb;       // K: r16 * k_row + 8 g4 (second half +32 bytes); 8 g4
  uint32_t ks;          // K scales: r16 * ks_row
  uint32_t v[4], vb;    // V: (4 g4 + i) * v_row + 4 r16; 4 r16
  uint32_t vs[4], vsb;  // V scales: (4 g4 + i) * vs_row + r16 / 2; r16 / 2
};

__device__ __forceinline__ LaneOffsetsN lane_offsetsN(const GqaParams& p, int r16, int g4) {
  LaneOffsetsN o;
  o.k = (uint32_t)r16 * (uint32_t)p.k_row + 8u * (uint32_t)g4;
  o.kb = 8u * (uint32_t)g4;
  o.ks = (uint32_t)r16 * (uint32_t)p.ks_row;
  for (int i = 0; i < 4; ++i) {
    o.v[i] = (uint32_t)(4 * g4 + i) * (uint32_t)p.v_row + 4u * (uint32_t)r16;
    o.vs[i] = (uint32_t)(4 * g4 + i) * (uint32_t)p.vs_row + (uint32_t)(r16 >> 1);
  }
  o.vb = 4u * (uint32_t)r16;
  o.vsb = (uint32_t)(r16 >> 1);
  return o;
}

// load_block for NVFP4 rows: 4 + 2 + 8 + 8 loads, same row clamping.
__device__ __forceinline__ RawBlockN load_blockN(const GqaParams& p, int g, int kb, int pg0, int pg1, int last_key,
                                                 int pmask, const LaneOffsetsN& lo) {
  RawBlockN r;
  for (int t = 0; t < 2; ++t) {
    const int st = min(kb + 16 * t, last_key);
    const uint32_t lim = (uint32_t)max(last_key - st, 0);
    const int64_t pg = t ? pg1 : pg0;
    const uint32_t row = (uint32_t)(st & pmask);
    const uint8_t* kbase = p.k + page_off(pg, p.k_page) + (int64_t)g * p.k_head + row * (uint32_t)p.k_row;
    const uint8_t* vbase = p.v + page_off(pg, p.v_page) + (int64_t)g * p.v_head + row * (uint32_t)p.v_row;
    const uint8_t* ksbase = p.ks + page_off(pg, p.ks_page) + (int64_t)g * p.ks_head + row * (uint32_t)p.ks_row;
    const uint8_t* vsbase = p.vs + page_off(pg, p.vs_page) + (int64_t)g * p.vs_head + row * (uint32_t)p.vs_row;
    const uint32_t koff = min(lo.k, lim * (uint32_t)p.k_row + lo.kb);
    r.k[t][0] = *reinterpret_cast<const uint2*>(kbase + koff);
    r.k[t][1] = *reinterpret_cast<const uint2*>(kbase + (koff + 32u));
    r.ks[t] = *reinterpret_cast<const uint2*>(ksbase + min(lo.ks, lim * (uint32_t)p.ks_row));
    const uint32_t vlim = lim * (uint32_t)p.v_row + lo.vb;
    const uint32_t vslim = lim * (uint32_t)p.vs_row + lo.vsb;
    for (int i = 0; i < 4; ++i) {
      r.v[4 * t + i] = *reinterpret_cast<const uint32_t*>(vbase + min(lo.v[i], vlim));
      r.vs[4 * t + i] = vsbase[min(lo.vs[i], vslim)];
    }
  }
  return r;
}

// Eight NVFP4 codes (element 2i in the low nibble of byte i) with their
// group scale -> the e4m3 bytes of e4m3(code * scale * 2^-3). The products
// are formed in f16, where they are exact: a code has at most two significant
// bits and s = scale / 8 at most four, with s in [2^-12, 56] (or 0), so every
// product is 0 or an f16 normal in [2^-13, 336]. Rounding that exact value to
// e4m3 (v_cvt_scalef32_pk_fp8_f16, round to nearest even, scale 1) gives the
// byte the f32 product gives: 12 VALU per 8 codes (codes -> f16 pairs, packed
// multiply, e4m3 pairs) instead of 16 through f32. Checked on the device for
// every code pair and scale byte: identical except that a -0 scale byte
// (which the quantiser never writes) yields +0 codes, an equal value.
__device__ __forceinline__ _Float16 nvfp4_scale_f16(uint32_t scale_byte) {
  return (_Float16)(__builtin_amdgcn_cvt_f32_fp8((int)scale_byte, 0) * 0.125f);  // exact
}

__device__ __forceinline__ uint2 nvfp4x8_to_e4m3(uint32_t codes, _Float16 s) {
  typedef short i16x2 __attribute__((ext_vector_type(2)));
  const f16x2 ss = {s, s};
  const f16x2 e01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * ss;
  const f16x2 e23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * ss;
  const f16x2 e45 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * ss;
  const f16x2 e67 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * ss;
  // each word is written by one conversion; the first one's other word is
  // its own (dead) input, so no zeroed register is needed
  i16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(__builtin_bit_cast(i16x2, e01), e01, 1.0f, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, e23, 1.0f, true);
  i16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(__builtin_bit_cast(i16x2, e45), e45, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(hi, e67, 1.0f, true);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

__device__ __forceinline__ RawBlock nvfp4_block_to_e4m3(const RawBlockN& c, int g4) {
  RawBlock r;
  for (int t = 0; t < 2; ++t)
    for (int h = 0; h < 2; ++h) {  // head dims 64 h + 16 g4 ..: group 4 h + g4
      const _Float16 sk = nvfp4_scale_f16(((h ? c.ks[t].y : c.ks[t].x) >> (8 * g4)) & 0xFFu);
      const uint2 lo = nvfp4x8_to_e4m3(c.k[t][h].x, sk);
      const uint2 hi = nvfp4x8_to_e4m3(c.k[t][h].y, sk);
      r.k[t][h] = uint4{lo.x, lo.y, hi.x, hi.y};
    }
  for (int j = 0; j < 8; ++j) r.v[j] = nvfp4x8_to_e4m3(c.v[j], nvfp4_scale_f16(c.vs[j]));
  return r;
}

// One 32-key block of packed fp6 K/V with an e4m3 query: S = K Q^T on the
// scaled MFMA (A format 2 = e2m3 or 3 = e3m2), then V converted to e4m3 and
// the fp8 softmax / PV.
template <int NB, bool QLDS, int KVF>
__device__ __forceinline__ void process_block_fp6(const RawBlock6& cur, int kb, const QOperand<NB>& q,
                                                  const uint8_t* qlds, const LaneOffsets6& lo, RowState<NB>& st,
                                                  const int* lim, int lim_min, float c2, int g4) {
  constexpr int kFmt = KVF == PKV_KV_E2M3 ? 2 : 3;
  const int lane = threadIdx.x & 63;
  if (QLDS) asm volatile("" ::: "memory");
  f32x4 sacc[NB][2];
  for (int t = 0; t < 2; ++t) {
    const i32x8 a = {(int)cur.k[t][0].x, (int)cur.k[t][0].y, (int)cur.k[t][1].x, (int)cur.k[t][1].y,
                     (int)cur.k[t][2].x, (int)cur.k[t][2].y, 0, 0};
    for (int nb = 0; nb < NB; ++nb) {
      long qv[4];
      for (int s = 0; s < 4; ++s)
        qv[s] = QLDS ? *reinterpret_cast<const long*>(qlds + ((4 * nb + s) * 64 + lane) * 8) : q.q8[nb][s];
      const i32x8 b = {(int)qv[0], (int)(qv[0] >> 32), (int)qv[1], (int)(qv[1] >> 32),
                       (int)qv[2], (int)(qv[2] >> 32), (int)qv[3], (int)(qv[3] >> 32)};
      // B format 0 = fp8 e4m3; E8M0 scales 127 = 2^0
      sacc[nb][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, kFmt, 0, 0,
                                                                      127, 0, 127);
    }
  }
  uint2 v8[8];
  fp6x32_to_e4m3<KVF>(cur.v, lo, v8);
  fp6x32_to_e4m3<KVF>(cur.v + 4, lo, v8 + 4);
  softmax_pv<true, NB, false>(sacc, v8, kb, st, lim, lim_min, c2, g4);
}

// Epilogue of one work item for kv head g of sequence b: a sequence with one
// split writes O and LSE itself; otherwise the rows go to split slot `slot`
// of the workspace for the merge kernel.
template <bool FP8Q, int NB>
__device__ __forceinline__ void finish_item(const GqaParams& p, const RowState<NB>& st, const RowMap<NB>& rm, int b,
                                            int g, int row0, int r16, int g4, int ns, int slot, float cs, float vdv) {
  const bool direct = ns <= 1;
  const float p_scale = FP8Q ? kP8Scale : 1.0f;
  int qtok[NB], qhead[NB];
  for (int nb = 0; nb < NB; ++nb) {
    qtok[nb] = b * p.q_len + rm.qi[nb];
    qhead[nb] = g * p.h_r + rm.hr[nb];
  }
  for (int nb = 0; nb < NB; ++nb) {
    const float l = wave_sum16(st.l_part[nb]) / p_scale;  // e4m3 P: l summed p * 448
    if (!rm.ok[nb]) continue;
    const int n = row0 + 16 * nb + r16;
    const int64_t stat_row = ((int64_t)b * p.h_k + g) * p.rows + n;
    const float m_nat = st.m_run[nb] == -INFINITY ? -INFINITY : st.m_run[nb] * cs;
    if (direct) {
      const float inv = l > 0.f ? (p.o_scale * vdv / p_scale) / l : 0.f;
      uint8_t* orow = p.o + (int64_t)qtok[nb] * p.o_tok + (int64_t)qhead[nb] * p.o_head;
      for (int i = 0; i < 4; ++i) {
        bf16x8 out;
        for (int mt = 0; mt < 8; ++mt) out[mt] = (__bf16)(st.oacc[nb][mt][i] * inv);
        *reinterpret_cast<bf16x8*>(orow + 2 * (32 * g4 + 8 * i)) = out;
      }
      if (g4 == 0) p.lse[stat_row] = l > 0.f ? m_nat + logf(l) : -INFINITY;
    } else {
      const int64_t prow = (int64_t)slot * p.num_seqs * p.h_k * p.rows + stat_row;
      const float ps = vdv / p_scale;
      float* dst = p.ws_o + prow * kD + 32 * g4;
      for (int i = 0; i < 4; ++i) {
        f32x4 lo4 = {st.oacc[nb][0][i], st.oacc[nb][1][i], st.oacc[nb][2][i], st.oacc[nb][3][i]};
        f32x4 hi4 = {st.oacc[nb][4][i], st.oacc[nb][5][i], st.oacc[nb][6][i], st.oacc[nb][7][i]};
        *reinterpret_cast<f32x4*>(dst + 8 * i) = lo4 * ps;
        *reinterpret_cast<f32x4*>(dst + 8 * i + 4) = hi4 * ps;
      }
      if (g4 == 0) p.ws_ml[prow] = float2{m_nat, l};
    }
  }
}

PKV_STAMP_STORAGE

#if PKV_STAMPS
// Stamped builds: wait until a block's loads have landed (an empty asm reads
// the register its last load fills, so the compiler's wait for it, which
// covers every earlier load, comes first).
__device__ __forceinline__ void landed(const RawBlock& r) { asm volatile("" ::"v"(r.v[7].x), "v"(r.v[7].y)); }
__device__ __forceinline__ void landed(const RawBlock4& r) { asm volatile("" ::"v"(r.v[7])); }
__device__ __forceinline__ void landed(const RawBlock6& r) { asm volatile("" ::"v"(r.v[7].x), "v"(r.v[7].y)); }
__device__ __forceinline__ void landed(const RawBlockN& r) { asm volatile("" ::"v"(r.vs[7])); }
#endif

// Load through the constant address space: with a wave-uniform address this
// is a scalar load, which completes out of order on its own counter, so
// waiting for it never waits for the KV loads in flight (a vector load
// would: those complete in order). For memory the kernel never writes.
template <typename T>
__device__ __forceinline__ T load_uniform(const T* ptr) {
  return *(const __attribute__((address_space(4))) T*)(ptr);
}
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clamp_page(const GqaParams& p, int pg) { return min(max(pg, 0), p.num_pages - 1); }

// Eight waves share four SIMDs: wave w and w ^ 4 sit on one SIMD, and the
// older wins issue by default. After each round a wave publishes how far it
// got (`done`, increasing) and runs at raised priority while it is not ahead
// of its sibling, so the two keep pace.
__device__ __forceinline__ void keep_pace(int* progress, int wave, int done, int lane) {
  if (lane == 0) __hip_atomic_store(progress + wave, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int sib = __hip_atomic_load(progress + (wave ^ 4), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (__builtin_amdgcn_readfirstlane(sib) >= done)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// One work item (a chunk of 128-key tiles of one sequence) for kv head g:
// the one-item-per-workgroup plan.
// KVF: 0 = e4m3 K/V, else the packed narrow format (PKV_KV_E2M1 fp4,
// PKV_KV_E2M3 / PKV_KV_E3M2 fp6, PKV_KV_NVFP4; e4m3 query only). The page pairs of a fetch
// are loaded LA fetches ahead: two for the e4m3 ring, one fewer than the ring
// depth for the deeper narrow rings (a pair loaded sooner would make its wait
// cover KV loads still in the ring).
template <bool FP8Q, int NB, bool CAUSAL_TAIL, int STAGES, int HW, int KVF = 0>
__device__ __forceinline__ void gqa_decode_item(const GqaParams& p, int item, int tile, int lane, int g, int* progress,
                                                int& round_base) {
  static_assert(KVF == 0 || FP8Q, "narrow K/V formats need the e4m3 query");
  constexpr int LA = KVF != 0 && STAGES > 2 ? STAGES - 1 : 2;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;

  const int4 w = p.work[item];
  const int b = w.x;
  if (w.z <= w.y || b < 0 || b >= p.num_seqs) return;  // padding item / bad entry
  const int page_size = 1 << p.page_shift;
  const int k_begin = w.y * p.key_mult;
  if (k_begin & (kBlockKeys - 1)) return;  // a key plan's items start on 32-key blocks (16-key groups stay in a page)
  // planned end of the chunk (the plan's lengths are upper bounds of the runtime ones)
  const int plan_last = min(w.z * p.key_mult, p.max_blocks * page_size) - 1;
  const int32_t* bt = p.block_table + (int64_t)b * p.bt_row;
  // Start-up: the page pairs of the first two fetches are read for the
  // planned chunk right away, so they travel with the sequence length, split
  // count, descales and query (one round trip where waiting for the length
  // first takes two). They are read again with the runtime bound below when
  // the length ends the chunk before the last of them. Entry indices stay in
  // [0, max_blocks) either way.
  auto plan_pair = [&](int kb) -> int {
    return bt[max(min(kb + 16 * (lane & 1), plan_last), 0) >> p.page_shift];
  };
  int pv[STAGES];
#pragma unroll
  for (int u = 0; u < LA; ++u) pv[u % STAGES] = plan_pair(k_begin + kBlockKeys * u);
  const int ns = p.n_splits[b];
  const int slot = w.w;
  int L = p.seq_lens[b];
  if (ns > 1 && (slot < 0 || slot >= p.max_splits)) return;
  const int row0 = tile * (16 * NB);

  L = max(0, min(L, p.max_blocks * page_size));
  const int k_end = min(plan_last + 1, L);

  const RowMap<NB> rm = row_map<NB>(p, row0, r16);
  int lim[NB];  // last key each row may see inside this work item's chunk
  for (int nb = 0; nb < NB; ++nb) lim[nb] = min(CAUSAL_TAIL ? L - p.q_len + rm.qi[nb] : L - 1, k_end - 1);
  const int lim_min = min(CAUSAL_TAIL ? L - p.q_len : L - 1, k_end - 1);

  const float qd = FP8Q ? p.qd[b * p.qd_seq + g * p.qd_head] : 1.0f;
  const float kdv = p.kd[b * p.kd_seq + g * p.kd_head];
  const float vdv = p.vd[b * p.vd_seq + g * p.vd_head];
  const float c2 = p.scale_log2e * qd * kdv;  // exponent scale (base 2) on raw scores
  const float cs = p.scale * qd * kdv;        // natural-log scale of the running max

  constexpr bool kQLds = NB == 2;
  extern __shared__ __attribute__((aligned(16))) uint8_t gqa_q_lds[];
  uint8_t* qlds = gqa_q_lds + (threadIdx.x >> 6) * (NB * 4 * 64 * (FP8Q ? 8 : 16));
  QOperand<NB> q;
  load_q<FP8Q, NB>(p, q, rm, b, g, g4);
  if (kQLds) park_q<FP8Q, NB>(q, qlds, lane);
  RowState<NB> st;
  reset_rows<NB>(st);

  if (k_end > k_begin) {
    const int last_key = k_end - 1;  // loads never go past the chunk (and so never past L)
    const int pmask = page_size - 1;
    // Pages of one 32-key block (page_size >= 16, so each 16-key group lies
    // in one page): lane l loads the entry of group l & 1, so lanes 0 and 1
    // hold the block's two pages. A vector load, so waiting for it (in
    // order) never waits for the KV loads issued after it.
    auto page_pair = [&](int kb) -> int { return bt[min(kb + 16 * (lane & 1), last_key) >> p.page_shift]; };

    // Fetch u loads block k_begin + 32u into ring slot u % STAGES. Every
    // fetch issues the same 13 loads whether or not its block exists (a
    // block past the chunk re-reads the chunk's last row, a cache hit), so
    // the compiler counts the loads in flight exactly and each wait covers
    // only the block being consumed. Fetch u takes its two pages from page
    // slot u % STAGES (loaded two fetches earlier) and loads the pages of
    // fetch u + 2 into slot (u + 2) % STAGES; slot indices are compile-time
    // constants of the unrolled stage loop.
    // the early pairs are right unless the length ends the chunk before the
    // last key they cover
    if (last_key < plan_last && last_key < k_begin + kBlockKeys * (LA - 1) + 16) {
#pragma unroll
      for (int u = 0; u < LA; ++u) pv[u % STAGES] = page_pair(k_begin + kBlockKeys * u);
    }
    constexpr bool kFp4 = KVF == PKV_KV_E2M1, kFp6 = KVF == PKV_KV_E2M3 || KVF == PKV_KV_E3M2;
    constexpr bool kNv = KVF == PKV_KV_NVFP4;
    using Raw = typename std::conditional<
        kFp4, RawBlock4,
        typename std::conditional<kFp6, RawBlock6,
                                  typename std::conditional<kNv, RawBlockN, RawBlock>::type>::type>::type;
    const auto lo = [&] {
      if constexpr (kFp4)
        return lane_offsets4(p, r16, g4);
      else if constexpr (kFp6)
        return lane_offsets6(p, r16, g4);
      else if constexpr (kNv)
        return lane_offsetsN(p, r16, g4);
      else
        return lane_offsets(p, r16, g4);
    }();
    auto fetch = [&](Raw& r, int kb, const int slot) {
      const int pg0 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 0));
      const int pg1 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 1));
      if constexpr (kFp4)
        r = load_block4(p, g, kb, pg0, pg1, last_key, pmask, lo);
      else if constexpr (kFp6)
        r = load_block6(p, g, kb, pg0, pg1, last_key, pmask, lo);
      else if constexpr (kNv)
        r = load_blockN(p, g, kb, pg0, pg1, last_key, pmask, lo);
      else
        r = load_block(p, g, kb, pg0, pg1, last_key, pmask, lo);
      pv[(slot + LA) % STAGES] = page_pair(kb + LA * kBlockKeys);
    };

    // Ring of STAGES register buffers: while block i is processed, blocks
    // i+1 .. i+STAGES-1 are in flight.
    // The loop runs whole rounds of STAGES blocks with no early exit, so
    // entry and back edge see the same loads in flight. Blocks past the
    // chunk (at most STAGES - 1 per work item) re-read its last row and are
    // masked out entirely (P = 0 on finite data): they change nothing.
    // The prologue's fetches stay in issue order (the scheduler would
    // otherwise hoist the later K loads past the page-pair loads, and the
    // wait at the loop header, shared by entry and back edge, would drain
    // the ring on every pass of the loop).
    Raw ring[STAGES];
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
      fetch(ring[s], k_begin + kBlockKeys * s, s);
      __builtin_amdgcn_sched_barrier(0);
    }
    const int rounds = (k_end - k_begin + kBlockKeys * STAGES - 1) / (kBlockKeys * STAGES);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int r = 0; r < rounds; ++r) {
      const int kb0 = k_begin + r * kBlockKeys * STAGES;
#pragma unroll
      for (int s = 0; s < STAGES; ++s) {
        const int kb = kb0 + kBlockKeys * s;
        // stamps (stamped builds): issue 0 -> 1, wait for the block 1 -> 2, processing 2 -> 3
        PKV_STAMP_VARS
        PKV_STAMP(0);
        fetch(ring[(s + STAGES - 1) % STAGES], kb + kBlockKeys * (STAGES - 1), (s + STAGES - 1) % STAGES);
        PKV_STAMP(1);
#if PKV_STAMPS
        landed(ring[s]);
#endif
        PKV_STAMP(2);
        if constexpr (kFp4)
          process_block_fp4<NB, kQLds>(ring[s], kb, q, qlds, st, lim, lim_min, c2, g4);
        else if constexpr (kFp6)
          process_block_fp6<NB, kQLds, KVF>(ring[s], kb, q, qlds, lo, st, lim, lim_min, c2, g4);
        else if constexpr (kNv)
          process_block<true, NB, kQLds>(nvfp4_block_to_e4m3(ring[s], g4), kb, q, qlds, st, lim, lim_min, c2, g4);
        else
          process_block<FP8Q, NB, kQLds>(ring[s], kb, q, qlds, st, lim, lim_min, c2, g4);
        PKV_STAMP(3);
        PKV_STAMP_SAVE(r * STAGES + s, round_base == 0);
      }
      if (HW == 8 && !p.paired) keep_pace(progress, wave, round_base + r, lane);
    }
    round_base += rounds;
  }
  finish_item<FP8Q, NB>(p, st, rm, b, g, row0, r16, g4, ns, slot, cs, vdv);
}

// Bytes of dynamic LDS per wave for the parked query of two row blocks.
template <bool FP8Q, int NB>
constexpr int q_park_bytes() {
  return NB == 2 ? NB * 4 * 64 * (FP8Q ? 8 : 16) : 0;
}

// V rows of keys past `vlast` (loaded through planned block-table entries
// that may lie past the sequence) are zeroed, so that P = 0 never meets a
// non-finite value in PV. Lane (r16, g4) holds in v[j] the key
// kb + 16 (j >> 2) + 4 g4 + (j & 3).
__device__ __forceinline__ void zero_tail_v(RawBlock& r, int kb, int vlast, int g4) {
  for (int j = 0; j < 8; ++j)
    if (kb + 16 * (j >> 2) + 4 * g4 + (j & 3) > vlast) r.v[j] = uint2{0u, 0u};
}

// Persistent form of the queued plan, one row block: wave (workgroup x, kv
// head g) runs the items of bin x, then items of kv head g's queue until it
// is empty. The items form ONE load stream. Each item runs whole rounds of
// STAGES 32-key blocks (at least two), as the one-item form does. The last
// round already fetches the next item N's first blocks, so an item boundary
// costs its epilogue and no round trip. N is prepared while the current item
// runs, with scalar loads only:
//   - at the item's start, take a queue item (once the bin is done);
//   - at the end of the third-to-last round, read N's work entry;
//   - at the end of the second-to-last round, its length, split count and
//     descales;
//   - in the last round, its query and first blocks.
// Every round therefore issues the same vector loads, and the compiler's
// waits stay exact. Block-table entries are loaded two fetches ahead, as in
// the one-item form, from the planned key range, which needs no sequence
// length. Rows past the runtime length are clamped to its last key, and
// their V is zeroed before use.
template <bool FP8Q, bool CAUSAL_TAIL, int STAGES, int HW>
__device__ __forceinline__ void gqa_decode_persistent(const GqaParams& p, int lane, int g, int* progress) {
  constexpr int NB = 1;
  constexpr int S = STAGES;
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int row0 = blockIdx.z * 16;
  const RowMap<NB> rm = row_map<NB>(p, row0, r16);
  const int page_size = 1 << p.page_shift;
  const int pmask = page_size - 1;
  const int key_cap = p.max_blocks * page_size;
  const LaneOffsets lo = lane_offsets(p, r16, g4);
  const int bin_hi = p.bin_offsets[blockIdx.x + 1];
  const int q0 = p.bin_offsets[gridDim.x];
  const int col = blockIdx.z * p.h_k + g;
  int* const taken = p.queue + col;                          // queue items handed out for this column
  int* const retired = p.queue + p.h_k * gridDim.z + col;    // waves of this column done taking
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  struct Meta {
    int idx, b, k_begin, plan_last, slot, ns, L;
    bool entry_ok;
    float qd, kd, vd;
  };
  auto load_entry = [&](Meta& m) {  // work entry of m.idx (any idx: the load is clamped)
    const i32x4 w = load_uniform(reinterpret_cast<const i32x4*>(p.work) + min(max(m.idx, 0), p.num_work - 1));
    m.entry_ok = m.idx < p.num_work && w.x >= 0 && w.x < p.num_seqs && w.y >= 0 && w.z > w.y;
    m.b = min(max(w.x, 0), p.num_seqs - 1);
    m.k_begin = max(w.y, 0);
    m.plan_last = max(min(w.z, key_cap) - 1, m.k_begin);  // planned last key (>= k_begin: an entry exists)
    m.slot = w.w;
  };
  auto load_seq = [&](Meta& m) {
    m.ns = load_uniform(p.n_splits + m.b);
    m.L = max(0, min(load_uniform(p.seq_lens + m.b), key_cap));
    m.qd = FP8Q ? load_uniform(p.qd + m.b * p.qd_seq + g * p.qd_head) : 1.0f;
    m.kd = load_uniform(p.kd + m.b * p.kd_seq + g * p.kd_head);
    m.vd = load_uniform(p.vd + m.b * p.vd_seq + g * p.vd_head);
  };
  auto last_key_of = [&](const Meta& m) {  // last key a load may touch (< k_begin: none)
    return m.entry_ok ? min(m.plan_last + 1, m.L) - 1 : m.k_begin - 1;
  };
  // At least two rounds per item (masked ones past its keys): the next item
  // is then always known before the round whose block-table entries reach
  // into it is loaded, and every round issues the same loads.
  auto rounds_of = [&](const Meta& m) {
    const int keys = last_key_of(m) + 1 - m.k_begin;
    return max(2, (keys + kBlockKeys * S - 1) / (kBlockKeys * S));
  };

  // current item C and the next item N
  Meta C, N;
  int grab = 0;  // lane 0: result of the last queue take
  auto take = [&]() {
    if (lane == 0) grab = __hip_atomic_fetch_add(taken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  const int bin_lo = p.bin_offsets[blockIdx.x];
  if (bin_lo < bin_hi) {
    C.idx = bin_lo;
  } else {
    take();
    C.idx = q0 + __builtin_amdgcn_readlane(grab, 0);
  }
  if (C.idx < p.num_work) {
    load_entry(C);
    load_seq(C);
    QOperand<NB> q, qn;
    load_q<FP8Q, NB>(p, q, rm, C.b, g, g4);
    bool n_valid = false;  // N exists and its entry has been read
    N.idx = p.num_work;

    int c_last = last_key_of(C), n_last = -1;
    // Page pair of fetch slot u (lanes 0 / 1: the pages of its two 16-key
    // groups) from the planned key range: C's slots below c_slots, N's at or
    // past it once N is known (nx_ok), else C's last block again.
    auto pair_of = [&](int u, int c_slots, bool nx_ok) -> int {
      const bool nx = nx_ok && u >= c_slots;
      const int bb = nx ? N.b : C.b;
      const int key = nx ? N.k_begin + kBlockKeys * (u - c_slots) : C.k_begin + kBlockKeys * u;
      const int kk = min(min(key + 16 * (lane & 1), nx ? N.plan_last : C.plan_last), key_cap - 1);
      return p.block_table[(int64_t)bb * p.bt_row + (max(kk, 0) >> p.page_shift)];
    };
    // Fetch slot u into `r` with the pair in pv[slot], and load the pair of
    // slot u + 2 into pv[(slot + 2) % S] (slot indices are compile-time
    // constants of the unrolled stage loop). fetch_n: slot u may be N's (N's
    // last key known); pair_n: slot u + 2 may be N's (N's entry known).
    int pv[S];
    auto fetch = [&](RawBlock& r, int u, int c_slots, bool fetch_n, bool pair_n, const int slot) {
      const bool nx = fetch_n && u >= c_slots;
      const int kb = nx ? N.k_begin + kBlockKeys * (u - c_slots) : C.k_begin + kBlockKeys * u;
      const int pg0 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 0));
      const int pg1 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 1));
      r = load_block(p, g, kb, pg0, pg1, nx ? n_last : c_last, pmask, lo);
      pv[(slot + 2) % S] = pair_of(u + 2, c_slots, pair_n);
    };

    int R = rounds_of(C);
    RawBlock ring[S];
    // first item: its first S - 1 blocks
    pv[0] = pair_of(0, R * S, false);
    pv[1 % S] = pair_of(1, R * S, false);
#pragma unroll
    for (int d = 0; d < S - 1; ++d) fetch(ring[d], d, R * S, false, false, d);
    int round_base = 0;
    for (;;) {
      // ---- current item C --------------------------------------------------
      const bool c_ok = C.entry_ok && (C.ns <= 1 || (C.slot >= 0 && C.slot < p.max_splits));
      int lim[NB];
      for (int nb = 0; nb < NB; ++nb) lim[nb] = min(CAUSAL_TAIL ? C.L - p.q_len + rm.qi[nb] : C.L - 1, c_last);
      const int lim_min = min(CAUSAL_TAIL ? C.L - p.q_len : C.L - 1, c_last);
      const float c2 = p.scale_log2e * C.qd * C.kd;
      const float cs = p.scale * C.qd * C.kd;
      const int c_slots = R * S;
      const bool n_static = C.idx + 1 < bin_hi;  // else N comes from the queue
      // a queue item for N is taken as C starts; its result is read, and N's
      // entry loaded, at the end of round R - 3 (at once for two-round items:
      // round 0 then already fetches N's first page pair)
      if (!n_static) take();
      auto prepare_n = [&]() {
        N.idx = n_static ? C.idx + 1 : q0 + __builtin_amdgcn_readlane(grab, 0);
        load_entry(N);
        n_valid = N.idx < p.num_work;
      };
      if (R == 2) prepare_n();
      RowState<NB> st;
      reset_rows<NB>(st);

      // rounds 0 .. R-2: C's blocks; N is prepared with scalar loads (its
      // entry 3 rounds before the end, its sequence 2 rounds before), so every
      // round issues the same vector loads
      for (int r = 0; r < R - 1; ++r) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          fetch(ring[(s + S - 1) % S], r * S + s + S - 1, c_slots, false, n_valid, (s + S - 1) % S);
          const int kb = C.k_begin + kBlockKeys * (r * S + s);
          if (kb + kBlockKeys - 1 > c_last) zero_tail_v(ring[s], kb, c_last, g4);
          process_block<FP8Q, NB, false>(ring[s], kb, q, nullptr, st, lim, lim_min, c2, g4);
        }
        if (HW == 8) keep_pace(progress, wave, round_base + r, lane);
        // at a round's end, so that many loads have been issued since the take
        if (r == R - 3) prepare_n();
        if (r == R - 2 && n_valid) load_seq(N);
      }
      {  // last round: N's query, and its first S - 1 blocks into the ring
        const int r = R - 1;
        if (n_valid) n_last = last_key_of(N);
        load_q<FP8Q, NB>(p, qn, rm, n_valid ? N.b : C.b, g, g4);
#pragma unroll
        for (int s = 0; s < S; ++s) {
          fetch(ring[(s + S - 1) % S], r * S + s + S - 1, c_slots, n_valid, n_valid, (s + S - 1) % S);
          const int kb = C.k_begin + kBlockKeys * (r * S + s);
          if (kb + kBlockKeys - 1 > c_last) zero_tail_v(ring[s], kb, c_last, g4);
          process_block<FP8Q, NB, false>(ring[s], kb, q, nullptr, st, lim, lim_min, c2, g4);
        }
        if (HW == 8) keep_pace(progress, wave, round_base + r, lane);
      }
      round_base += R;
      if (c_ok) finish_item<FP8Q, NB>(p, st, rm, C.b, g, row0, r16, g4, C.ns, C.slot, cs, C.vd);
      if (!n_valid) break;
      // ---- N becomes current: its first S - 1 blocks are in the ring and the
      // pairs of its next fetches in pv
      C = N;
      q = qn;
      c_last = n_last;
      R = rounds_of(C);
      n_valid = false;
      N.idx = p.num_work;
    }
  }
  // The wave of this column that retires last has seen every other one
  // finish taking, so nobody reads the counters again in this launch: it
  // clears both for the next launch.
  if (lane == 0 &&
      __hip_atomic_fetch_add(retired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
    __hip_atomic_store(taken, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(retired, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The work items of one bin of the balanced plan (key ranges of one or more
// sequences, in order) for kv head g, streamed through ONE ring: the loads of
// the next item's first blocks are in flight while the current item's last
// blocks are processed, so an item boundary costs its epilogue and nothing
// else.
//
// The bin's items are described by a table held one item per lane (up to 64
// items at a time): sequence, first key, clamped end, and the running count
// of 32-key blocks. Bin block j belongs to the item whose running count
// first exceeds j, found with one ballot and a popcount, and item fields are
// read with readlane -- no LDS, no scalar loads in the loop. Each item's
// query rows are loaded while the item before it runs.
template <bool FP8Q, int NB, bool CAUSAL_TAIL, int STAGES, int HW>
__device__ __forceinline__ void gqa_decode_stream(const GqaParams& p, int lane, int g, int* progress) {
  const int r16 = lane & 15;
  const int g4 = lane >> 4;
  const int row0 = blockIdx.z * (16 * NB);
  const int page_size = 1 << p.page_shift;
  const int pmask = page_size - 1;
  const int key_cap = p.max_blocks * page_size;
  const RowMap<NB> rm = row_map<NB>(p, row0, r16);
  const LaneOffsets lo = lane_offsets(p, r16, g4);
  const int it_lo = p.bin_offsets[blockIdx.x];
  const int it_hi = p.bin_offsets[blockIdx.x + 1];

  for (int seg = it_lo; seg < it_hi; seg += 64) {
    const int np = min(64, it_hi - seg);
    // ---- item table: lane i describes item seg + i ---------------------------
    int t_b = 0, t_k0 = 0, t_end = 0, t_L = 0, t_slot = 0, t_ns = 1, t_ok = 0, nblk = 0;
    float t_kd = 0.f, t_vd = 0.f, t_qd = 1.f;
    if (lane < np) {
      const int4 w = p.work[seg + lane];
      if (w.x >= 0 && w.x < p.num_seqs && w.y >= 0 && w.z >= w.y) {
        t_b = w.x;
        t_k0 = w.y;
        t_L = max(0, min(p.seq_lens[t_b], key_cap));
        t_end = min(w.z, t_L);
        t_ns = p.n_splits[t_b];
        t_slot = w.w;
        t_ok = t_ns <= 1 || (t_slot >= 0 && t_slot < p.max_splits);
        // blocks of the planned range; keys past L are loaded clamped and masked
        nblk = t_ok ? (min(w.z, key_cap) - w.y + kBlockKeys - 1) / kBlockKeys : 0;
        nblk = max(nblk, 0);
        t_kd = p.kd[t_b * p.kd_seq + g * p.kd_head];
        t_vd = p.vd[t_b * p.vd_seq + g * p.vd_head];
        if (FP8Q) t_qd = p.qd[t_b * p.qd_seq + g * p.qd_head];
      }
    }
    int cum = nblk;  // inclusive running count of blocks over the items
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(cum, d, 64);
      if (lane >= d) cum += o;
    }
    const int nblocks = __builtin_amdgcn_readlane(cum, 63);
    const int cum_end = lane < np ? cum : 0x7fffffff;
    const int t_kbase = t_k0 - kBlockKeys * (cum - nblk);  // key of bin block j = t_kbase + 32 j
    const int t_last = max(t_end - 1, 0);                   // loads clamp to this key (< L when L > 0)
    auto item_of = [&](int j) -> int {  // the item holding bin block j < nblocks
      return (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(cum_end <= j));
    };

    // ---- current item ----------------------------------------------------------
    QOperand<NB> qc, qn;  // query rows of the current item / of the next one
    RowState<NB> st;
    reset_rows<NB>(st);
    int cur = -1;
    int c_b = 0, c_ns = 1, c_slot = 0, c_ok = 0, lim_min = -1, lim_max = -1;
    int lim[NB];
    for (int nb = 0; nb < NB; ++nb) lim[nb] = -1;
    float c2 = 0.f, cs = 0.f, c_vd = 0.f;
    auto prefetch_q = [&](int i) {
      if (i < np) load_q<FP8Q, NB>(p, qn, rm, __builtin_amdgcn_readlane(t_b, i), g, g4);
    };
    auto begin_item = [&](int i) {
      qc = qn;
      c_b = __builtin_amdgcn_readlane(t_b, i);
      c_ns = __builtin_amdgcn_readlane(t_ns, i);
      c_slot = __builtin_amdgcn_readlane(t_slot, i);
      c_ok = __builtin_amdgcn_readlane(t_ok, i);
      const int L = __builtin_amdgcn_readlane(t_L, i);
      const int k_end = __builtin_amdgcn_readlane(t_end, i);
      for (int nb = 0; nb < NB; ++nb) lim[nb] = min(CAUSAL_TAIL ? L - p.q_len + rm.qi[nb] : L - 1, k_end - 1);
      lim_min = min(CAUSAL_TAIL ? L - p.q_len : L - 1, k_end - 1);
      lim_max = k_end - 1;
      const float qd = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(t_qd), i));
      const float kd = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(t_kd), i));
      c_vd = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(t_vd), i));
      c2 = p.scale_log2e * qd * kd;
      cs = p.scale * qd * kd;
      reset_rows<NB>(st);
      prefetch_q(i + 1);
    };
    auto end_item = [&]() {
      if (c_ok) finish_item<FP8Q, NB>(p, st, rm, c_b, g, row0, r16, g4, c_ns, c_slot, cs, c_vd);
    };
    auto advance_to = [&](int i) {  // finish items before i (empty ones too), begin item i
      while (cur < i) {
        if (cur >= 0) end_item();
        ++cur;
        begin_item(cur);
      }
    };
    prefetch_q(0);

    if (nblocks > 0) {
      // bin block j (clamped to the last one: blocks past the bin re-read it)
      auto block_at = [&](int j, int& b, int& kb, int& last) {
        const int jc = min(j, nblocks - 1);
        const int i = item_of(jc);
        b = __builtin_amdgcn_readlane(t_b, i);
        kb = __builtin_amdgcn_readlane(t_kbase, i) + kBlockKeys * jc;
        last = __builtin_amdgcn_readlane(t_last, i);
      };
      auto page_pair = [&](int j) -> int {  // lanes 0 / 1: pages of the block's two 16-key groups
        int b, kb, last;
        block_at(j, b, kb, last);
        return p.block_table[(int64_t)b * p.bt_row + (min(kb + 16 * (lane & 1), last) >> p.page_shift)];
      };
      // Same discipline as the one-item path: every step issues the same
      // loads, page pairs two fetches ahead in a vector ring.
      int pv[STAGES];
      pv[0] = page_pair(0);
      pv[1 % STAGES] = page_pair(1);
      auto fetch = [&](RawBlock& r, int j, const int slot) {
        int b, kb, last;
        block_at(j, b, kb, last);
        const int pg0 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 0));
        const int pg1 = clamp_page(p, __builtin_amdgcn_readlane(pv[slot], 1));
        r = load_block(p, g, kb, pg0, pg1, last, pmask, lo);
        pv[(slot + 2) % STAGES] = page_pair(j + 2);
      };
      RawBlock ring[STAGES];
#pragma unroll
      for (int s = 0; s < STAGES - 1; ++s) fetch(ring[s], s, s);
      const int rounds = (nblocks + STAGES - 1) / STAGES;
      const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
      for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int s = 0; s < STAGES; ++s) {
          const int j = r * STAGES + s;
          fetch(ring[(s + STAGES - 1) % STAGES], j + STAGES - 1, (s + STAGES - 1) % STAGES);
          if (j < nblocks) {
            const int i = item_of(j);
            if (i != cur) advance_to(i);
            const int kb = __builtin_amdgcn_readlane(t_kbase, i) + kBlockKeys * j;
            // a block with no key below the item's end (past L) is skipped
            if (kb <= lim_max) process_block<FP8Q, NB, false>(ring[s], kb, qc, nullptr, st, lim, lim_min, c2, g4);
          }
        }
        if (HW == 8) keep_pace(progress, wave, seg * 65536 + r, lane);
      }
    }
    advance_to(np - 1);  // items after the last block (empty ones)
    end_item();
  }
}

// Persistent form of two row blocks (queued plan): the items of this
// workgroup's bin, then items of the shared queue of its (kv-head group,
// q-row tile) until it is empty, each started afresh with the one-item
// loop. Every wave of the workgroup runs the same items (one kv head each)
// and meets the same barriers.
template <bool FP8Q, int NB, bool CAUSAL_TAIL, int STAGES, int HW>
__device__ __forceinline__ void gqa_decode_bin_then_queue(const GqaParams& p, int lane, int g, int* progress) {
  int round_base = 0;
  const int it_end = p.bin_offsets[blockIdx.x + 1];
  for (int it = p.bin_offsets[blockIdx.x]; it < it_end; ++it)
    if (g < p.h_k) gqa_decode_item<FP8Q, NB, CAUSAL_TAIL, STAGES, HW>(p, it, blockIdx.z, lane, g, progress, round_base);
  const int q0 = p.bin_offsets[gridDim.x];
  const int col = blockIdx.z * gridDim.y + blockIdx.y;         // < h_k * q tiles
  int* const taken = p.queue + col;                            // queue items handed out (+ one per final take)
  int* const retired = p.queue + gridDim.y * gridDim.z + col;  // workgroups done taking
  // the taken index, shared through the dynamic LDS past the parked queries
  extern __shared__ __attribute__((aligned(16))) uint8_t gqa_q_lds[];
  int& next_item = *reinterpret_cast<int*>(gqa_q_lds + HW * q_park_bytes<FP8Q, NB>());
  for (;;) {
    if (threadIdx.x == 0)
      next_item = q0 + __hip_atomic_fetch_add(taken, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int it = __builtin_amdgcn_readfirstlane(next_item);
    __syncthreads();  // everyone has read next_item before it is written again
    if (it >= p.num_work) break;
    if (g < p.h_k) gqa_decode_item<FP8Q, NB, CAUSAL_TAIL, STAGES, HW>(p, it, blockIdx.z, lane, g, progress, round_base);
  }
  // The workgroup that retires last has seen every other one finish taking,
  // so nobody reads the counters again in this launch: it clears both for the
  // next launch.
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(retired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
    __hip_atomic_store(taken, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(retired, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// HW waves per workgroup, one per kv head of the same work item: together
// they stream the same pages (every head's rows of a key range), which keeps
// the number of concurrent DRAM streams per key range at two (K, V). A
// workgroup runs one work item, or with a balanced plan the items of its
// bin (a contiguous share of all sequences' keys) as one stream.
// Capped at two waves per SIMD (256 registers), which keeps the compiler from
// parking values in AGPRs when the workgroup would allow one wave per SIMD:
// one row block fits as is, two row blocks of the one-item form fit with the
// query in LDS. The streaming form of two row blocks gets the whole file.
// Workgroup id -> (work item, q-row tile) so that the tiles of one item get
// ids i, i + 8, i + 16, ...: consecutive ids go to the 8 XCDs in turn, so
// an item's tiles run at about the same time on one XCD and the later ones
// read the item's pages from that XCD's L2.
__device__ __forceinline__ void xcd_item_tile(int id, int units, int tiles, int& unit, int& tile) {
  constexpr int kXcds = 8;
  const int chunk = id / (kXcds * tiles);
  const int local = id - chunk * kXcds * tiles;
  const int left = min(kXcds, units - chunk * kXcds);
  unit = chunk * kXcds + local % left;
  tile = local / left;
}

// Rounds done per wave, for the eight-wave workgroups that keep their two
// waves per SIMD in step; no LDS in the other forms (whose dynamic LDS may
// take all of the CU's).
template <int HW>
__device__ __forceinline__ int* wave_progress() {
  if constexpr (HW == 8) {
    __shared__ int progress[8];
    return progress;
  } else {
    return nullptr;
  }
}

template <bool FP8Q, int NB, bool CAUSAL_TAIL, int STAGES, int HW, bool STREAM, int KVF = 0>
__global__ __launch_bounds__(64 * HW) __attribute__((amdgpu_waves_per_eu(NB == 1 || !STREAM ? 2 : 1)))
void gqa_decode_kernel(GqaParams p) {
  const int lane = threadIdx.x & 63;
  int* const progress = wave_progress<HW>();
  if constexpr (HW == 8) {
    if (lane == 0) progress[threadIdx.x >> 6] = -1;
    __syncthreads();
  }
  int g = __builtin_amdgcn_readfirstlane(blockIdx.y * HW + (threadIdx.x >> 6));  // wave-uniform
  // one-item form: the work item and q-row tile of this workgroup
  int item = blockIdx.x, tile = blockIdx.z;
  if (p.xcd_tiles) xcd_item_tile(blockIdx.x, p.num_work, p.q_tiles, item, tile);
  if (HW == 8 && p.paired) {  // paired plan: waves 0-3 run item 2x, waves 4-7 item 2x + 1 (kv heads 0-3 each)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    item = 2 * blockIdx.x + (wave >> 2);
    g = wave & 3;
  }
  if constexpr (KVF != 0) {  // packed narrow K/V: the one-item form
    int round_base = 0;
    if (g < p.h_k) gqa_decode_item<FP8Q, NB, CAUSAL_TAIL, STAGES, HW, KVF>(p, item, tile, lane, g, progress, round_base);
    return;
  }
  if (STREAM) {
    if (g < p.h_k) gqa_decode_stream<FP8Q, NB, CAUSAL_TAIL, STAGES, HW>(p, lane, g, progress);
    return;
  }
  if (!p.queue) {
    int round_base = 0;
    if (g < p.h_k) gqa_decode_item<FP8Q, NB, CAUSAL_TAIL, STAGES, HW>(p, item, tile, lane, g, progress, round_base);
    return;
  }
  // queued plan: persistent workgroups
  if constexpr (NB == 1) {
    if (g < p.h_k) gqa_decode_persistent<FP8Q, CAUSAL_TAIL, STAGES, HW>(p, lane, g, progress);
  } else {
    gqa_decode_bin_then_queue<FP8Q, NB, CAUSAL_TAIL, STAGES, HW>(p, lane, g, progress);
  }
}

// Ring depth in 32-key blocks. Three blocks (two in flight while one is
// processed), except for the one-item form of two row blocks: with three
// blocks it needs more than 256 VGPRs, and the compiler then shuttles the O
// accumulators through AGPRs on every block. Two blocks plus the query in
// LDS fit in 256 registers, so two waves can share a SIMD (measured on
// the speculative-verify workload: 99.2 -> 96.3 us).
template <int NB, bool STREAM>
constexpr int ring_stages() {
  return (NB == 2 && !STREAM) ? 2 : 3;
}

template <bool FP8Q, int NB, bool CT, int HW>
const void* kernel_ptr(bool stream) {
  return stream ? reinterpret_cast<const void*>(&gqa_decode_kernel<FP8Q, NB, CT, ring_stages<NB, true>(), HW, true>)
                : reinterpret_cast<const void*>(&gqa_decode_kernel<FP8Q, NB, CT, ring_stages<NB, false>(), HW, false>);
}

// Packed narrow K/V: one-item form. One row block: a ring of three 4 KB fp4
// blocks (measured on the fully-fp8 batch with fp4 K/V, ring depths 2-5:
// 106.8, 105.0, 109.2, 110.6 us) or four 6 KB fp6 blocks (fp6's 15 loads
// per fetch also bound its depth); two row blocks: three (fp4) or two (fp6,
// whose conversion needs the registers a third block would take).
#ifndef PKV_FP4_STAGES
#define PKV_FP4_STAGES 3
#endif
#ifndef PKV_FP6_STAGES
#define PKV_FP6_STAGES 4
#endif
// NVFP4, one row block: two blocks (at two waves per SIMD, its plan: 155.6
// against 164 us with three)
#ifndef PKV_NV_STAGES
#define PKV_NV_STAGES 2
#endif
template <int NB, int KVF>
constexpr int narrow_stages() {
  // NVFP4: 23 loads per fetch, so at most two fetches ahead (the load counter holds 63)
  return KVF == PKV_KV_NVFP4 ? (NB == 2 ? 2 : PKV_NV_STAGES)
                             : NB == 2 ? (KVF == PKV_KV_E2M1 ? 3 : 2) : KVF == PKV_KV_E2M1 ? PKV_FP4_STAGES : PKV_FP6_STAGES;
}

template <int NB, bool CT, int HW, int KVF>
const void* narrow_ptr() {
  return reinterpret_cast<const void*>(&gqa_decode_kernel<true, NB, CT, narrow_stages<NB, KVF>(), HW, false, KVF>);
}

template <int NB, bool CT, int KVF>
const void* select_narrow_heads(const GqaVariant& v) {
  switch (v.heads_per_wg) {
    case 1: return narrow_ptr<NB, CT, 1, KVF>();
    case 2: return narrow_ptr<NB, CT, 2, KVF>();
    case 4: return narrow_ptr<NB, CT, 4, KVF>();
    default: return narrow_ptr<NB, CT, NB == 1 ? 8 : 4, KVF>();
  }
}

template <int KVF>
const void* select_narrow(const GqaVariant& v) {
  if (v.n_blocks == 1)
    return v.causal_tail ? select_narrow_heads<1, true, KVF>(v) : select_narrow_heads<1, false, KVF>(v);
  return v.causal_tail ? select_narrow_heads<2, true, KVF>(v) : select_narrow_heads<2, false, KVF>(v);
}

template <bool FP8Q, int NB, bool CT>
const void* select_heads(const GqaVariant& v) {
  switch (v.heads_per_wg) {
    case 1: return kernel_ptr<FP8Q, NB, CT, 1>(v.stream);
    case 2: return kernel_ptr<FP8Q, NB, CT, 2>(v.stream);
    case 4: return kernel_ptr<FP8Q, NB, CT, 4>(v.stream);
    default: return kernel_ptr<FP8Q, NB, CT, NB == 1 ? 8 : 4>(v.stream);
  }
}

template <bool FP8Q, int NB>
const void* select_tail(const GqaVariant& v) {
  return v.causal_tail ? select_heads<FP8Q, NB, true>(v) : select_heads<FP8Q, NB, false>(v);
}

const void* select_kernel(const GqaVariant& v) {
  if (v.kvf == PKV_KV_E2M1) return select_narrow<PKV_KV_E2M1>(v);
  if (v.kvf == PKV_KV_E2M3) return select_narrow<PKV_KV_E2M3>(v);
  if (v.kvf == PKV_KV_E3M2) return select_narrow<PKV_KV_E3M2>(v);
  if (v.kvf == PKV_KV_NVFP4) return select_narrow<PKV_KV_NVFP4>(v);
  if (v.fp8_q) return v.n_blocks == 1 ? select_tail<true, 1>(v) : select_tail<true, 2>(v);
  return v.n_blocks == 1 ? select_tail<false, 1>(v) : select_tail<false, 2>(v);
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

GqaVariant gqa_variant(const pkv_decode_args& a) {
  GqaVariant v;
  v.fp8_q = a.q_format == PKV_Q_E4M3;
  v.kvf = narrow_kv(a.kv_format) ? a.kv_format : 0;
  const int rows = a.q_len * (a.h_q / a.h_k);
  // two 16-row blocks per wave up to 32 rows: splitting them over two
  // workgroups (one block per wave) measured 124 vs 96 us on the
  // speculative-verify workload
  v.n_blocks = rows <= 16 ? 1 : 2;
  v.causal_tail = a.causal && a.q_len > 1;
  v.stream = a.bin_offsets != nullptr && a.queue == nullptr;
  if (v.kvf == PKV_KV_E2M1)
    v.stages = v.n_blocks == 1 ? narrow_stages<1, PKV_KV_E2M1>() : narrow_stages<2, PKV_KV_E2M1>();
  else if (v.kvf == PKV_KV_NVFP4)
    v.stages = v.n_blocks == 1 ? narrow_stages<1, PKV_KV_NVFP4>() : narrow_stages<2, PKV_KV_NVFP4>();
  else if (v.kvf)
    v.stages = v.n_blocks == 1 ? narrow_stages<1, PKV_KV_E2M3>() : narrow_stages<2, PKV_KV_E2M3>();
  else
    v.stages = (v.n_blocks == 2 && !v.stream) ? 2 : 3;
  // kv heads per workgroup: the largest power of two dividing h_k, up to 8
  // (4 for two row blocks: eight waves of 32 rows per workgroup measured
  // slower on the speculative-verify workload, 100 vs 95 us)
  const int cap = v.n_blocks == 1 ? 8 : 4;
  v.heads_per_wg = 1;
  while (v.heads_per_wg * 2 <= cap && a.h_k % (v.heads_per_wg * 2) == 0) v.heads_per_wg *= 2;
  // paired plan (four kv heads, one row block): eight waves, two items
  v.paired = a.work_pairs != 0;
  if (v.paired) v.heads_per_wg = 8;
  return v;
}

int gqa_rows_per_tile(const GqaVariant& v) { return 16 * v.n_blocks; }

// dynamic LDS of a variant: the parked query of two row blocks (one-item
// form), then, for e4m3 K/V, the queued form's shared word
size_t gqa_dyn_lds(const GqaVariant& v) {
  if (v.n_blocks != 2 || v.stream) return 0;
  return (size_t)v.heads_per_wg * 2 * 4 * 64 * (v.fp8_q ? 8 : 16) + (v.kvf == 0 ? 16 : 0);
}

hipError_t gqa_occupancy(const GqaVariant& v, int* units_per_cu) {
  // Units (work item, kv head, q tile) = waves. The plan is sized for about
  // four streaming waves per CU (at least one workgroup), not for the
  // register-limited maximum: per-CU read bandwidth saturates at ~32-64 KB
  // in flight, and a second workgroup on some CUs but not on others leaves
  // those CUs with twice the bytes (measured on the fully-fp8 workload:
  // 0.61 -> 0.68 of peak).
  int wgs = 0;
  const hipError_t e =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&wgs, select_kernel(v), 64 * v.heads_per_wg, gqa_dyn_lds(v));
  const int resident = wgs * v.heads_per_wg;
  // fp6 and NVFP4 K/V: eight units (two waves per SIMD), so that one wave's
  // conversions overlap the other's load waits (measured on the fully-fp8
  // batch: e2m3 K/V 178 -> 168 us, NVFP4 K/V 199.5 -> 162 us for the
  // kernel; fp4 K/V and e4m3 K/V gain nothing or lose)
  const bool two_waves = v.kvf == PKV_KV_E2M3 || v.kvf == PKV_KV_E3M2 || v.kvf == PKV_KV_NVFP4;
  const int target = v.heads_per_wg > 4 ? v.heads_per_wg : (two_waves ? 8 : 4);
  *units_per_cu = resident < target ? resident : target;
  return e;
}

hipError_t gqa_launch(const pkv_decode_args& a, const GqaVariant& v, hipStream_t stream) {
  GqaParams p;
  const int64_t qe = a.q_format == PKV_Q_BF16 ? 2 : 1;
  p.q = static_cast<const uint8_t*>(a.q);
  p.q_tok = a.q_tok_stride * qe;
  p.q_head = a.q_head_stride * qe;
  p.k = a.k;
  p.k_page = a.k_page_stride;
  p.k_row = a.k_row_stride;
  p.k_head = a.k_head_stride;
  p.v = a.v;
  p.v_page = a.v_page_stride;
  p.v_row = a.v_row_stride;
  p.v_head = a.v_head_stride;
  p.block_table = a.block_table;
  p.bt_row = a.bt_row_stride;
  p.seq_lens = a.seq_lens;
  p.qd = a.q_descale ? a.q_descale : a.k_descale;  // unused for bf16 q
  p.qd_seq = a.q_descale ? a.qd_seq_stride : 0;
  p.qd_head = a.q_descale ? a.qd_head_stride : 0;
  p.kd = a.k_descale;
  p.kd_seq = a.kd_seq_stride;
  p.kd_head = a.kd_head_stride;
  p.vd = a.v_descale;
  p.vd_seq = a.vd_seq_stride;
  p.vd_head = a.vd_head_stride;
  p.o = static_cast<uint8_t*>(a.o);
  p.o_tok = a.o_tok_stride * 2;
  p.o_head = a.o_head_stride * 2;
  p.lse = a.lse;
  p.work = reinterpret_cast<const int4*>(a.work);
  p.n_splits = a.n_splits;
  const int64_t rows_all = ws_rows(a);
  p.ws_o = static_cast<float*>(a.workspace);
  p.ws_ml = a.workspace ? reinterpret_cast<float2*>(p.ws_o + (int64_t)a.max_splits * rows_all * kD) : nullptr;
  p.bin_offsets = a.bin_offsets;
  p.queue = a.queue;
  p.ks = a.k_group_scale;
  p.ks_page = a.kgs_page_stride;
  p.ks_row = a.kgs_row_stride;
  p.ks_head = a.kgs_head_stride;
  p.vs = a.v_group_scale;
  p.vs_page = a.vgs_page_stride;
  p.vs_row = a.vgs_row_stride;
  p.vs_head = a.vgs_head_stride;
  p.key_mult = ((a.bin_offsets && a.queue) || a.work_in_keys) ? 1 : kTileKeys;
  p.num_work = a.num_work;
  p.scale_log2e = (float)((double)a.softmax_scale * 1.4426950408889634);
  p.scale = a.softmax_scale;
  p.o_scale = a.o_scale;
  p.num_seqs = a.num_seqs;
  p.q_len = a.q_len;
  p.h_k = a.h_k;
  p.h_r = a.h_q / a.h_k;
  p.rows = a.q_len * p.h_r;
  p.page_shift = log2_exact(a.page_size);
  p.num_pages = a.num_pages;
  p.max_blocks = a.max_blocks;
  p.max_splits = a.max_splits;
  const int tiles = (p.rows + gqa_rows_per_tile(v) - 1) / gqa_rows_per_tile(v);
  const int hw = v.heads_per_wg;
  p.q_tiles = tiles;
  p.xcd_tiles = !a.bin_offsets && tiles > 1;
  p.paired = v.paired ? 1 : 0;
  dim3 grid(a.bin_offsets ? a.num_bins : a.num_work, (a.h_k + hw - 1) / hw, tiles);  // bins: balanced or queued plan
  if (p.xcd_tiles) grid = dim3(a.num_work * tiles, (a.h_k + hw - 1) / hw, 1);
  if (v.paired) grid = dim3(a.num_work / 2, 1, 1);  // one q-row tile (16 rows), two items per workgroup
  void* args[] = {&p};
  const void* kernel = select_kernel(v);
  if (const hipError_t e = check_lds(kernel, gqa_dyn_lds(v)); e != hipSuccess) return e;
  return hipLaunchKernel(kernel, grid, dim3(64 * hw), args, gqa_dyn_lds(v), stream);
}

// stamps of the one-item loop (stamped builds; hipErrorNotSupported otherwise)
hipError_t gqa_copy_stamps(void* host_dst) { return PKV_STAMP_COPY(host_dst); }

}  // namespace pkv
