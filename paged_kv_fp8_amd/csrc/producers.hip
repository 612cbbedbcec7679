// The producers either side of the decode, for gfx950: the per-(sequence, kv
// head) e4m3 quantisation of the query and the write of new tokens into the
// paged KV cache (e4m3 rows with per-(sequence, kv head) descales, or latent
// records with per-token, per-128-value block scales).
//
// Method: "mjolnir-kernel 0.1.0 wheel: mjolnir/t5_decode.py", quantize_q_fp8
// (the largest |q| over a sequence's tokens, the kv head's query heads and d,
// at least 1e-6, over 448 is the descale; codes are the e4m3fn cast of
// q / descale) and its harness's KV pool (codes of x / descale per kv head);
// the page names the KV-cache write among the kernels that run before the
// decode without printing it. The write places the n_new newest tokens of a
// sequence at positions L - n_new .. L - 1 through the block table, and
// saturates values beyond the e4m3 range at +-448 (NaN stays NaN).
//
// gfx950 design: fp32 division (correctly rounded, as the cast's reference
// computes it), then the hardware e4m3 convert (round to nearest even) on a
// value already clamped to +-448, so overflow behaviour never matters.
// Loads are 16 bytes of bf16 per lane, stores 8 bytes of codes.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr float kE4m3Max = 448.0f;
constexpr float kMinAmax = 1e-6f;

// e4m3fn code of one fp32 value: NaN -> 0x7F, |x| > 448 -> +-448, else round
// to nearest even
__device__ __forceinline__ unsigned encode_one(float y) {
  if (y != y) return 0x7Fu;
  const float c = fminf(fmaxf(y, -kE4m3Max), kE4m3Max);
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// eight codes of eight values, packed little-endian into a uint2
__device__ __forceinline__ uint2 encode8(const float* y) {
  unsigned lo = 0, hi = 0;
  for (int e = 0; e < 4; ++e) lo |= encode_one(y[e]) << (8 * e);
  for (int e = 0; e < 4; ++e) hi |= encode_one(y[4 + e]) << (8 * e);
  return uint2{lo, hi};
}

__device__ __forceinline__ void unpack8(uint4 v, float* x) {
  const unsigned w[4] = {v.x, v.y, v.z, v.w};
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---- query quantisation: one workgroup per (sequence, kv head) --------------
struct QuantQParams {
  const uint8_t* q;  // bf16
  int64_t q_tok, q_head;  // bytes
  uint8_t* q8;
  int64_t q8_tok, q8_head;  // bytes
  float* qd;
  int64_t qd_seq, qd_head;  // elements
  int q_len, h_r, d;
};

__global__ __launch_bounds__(256) void quantize_q_kernel(QuantQParams p) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int d8 = p.d / 8;
  const int n = p.q_len * p.h_r * d8;  // 8-value pieces of the group
  auto piece = [&](int i, int& tok, int& head, int& off) {
    const int r = i / d8;  // row = (qi, hr), qi-major
    off = 8 * (i - r * d8);
    const int qi = r / p.h_r;
    tok = b * p.q_len + qi;
    head = g * p.h_r + (r - qi * p.h_r);
  };
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int tok, head, off;
    piece(i, tok, head, off);
    float x[8];
    unpack8(*reinterpret_cast<const uint4*>(p.q + (int64_t)tok * p.q_tok + (int64_t)head * p.q_head + 2 * off), x);
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  }
  __shared__ float part[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])), kMinAmax);
  const float descale = amax / kE4m3Max;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    int tok, head, off;
    piece(i, tok, head, off);
    float x[8];
    unpack8(*reinterpret_cast<const uint4*>(p.q + (int64_t)tok * p.q_tok + (int64_t)head * p.q_head + 2 * off), x);
    for (int e = 0; e < 8; ++e) x[e] = x[e] / descale;
    *reinterpret_cast<uint2*>(p.q8 + (int64_t)tok * p.q8_tok + (int64_t)head * p.q8_head + off) = encode8(x);
  }
  if (threadIdx.x == 0) p.qd[b * p.qd_seq + g * p.qd_head] = descale;
}

// ---- e4m3 cache write: 16 threads per (new token, kv head) row of d <= 128 ---
struct WriteKvParams {
  const uint8_t* k_new;  // bf16
  int64_t kn_tok, kn_head;  // bytes
  const uint8_t* v_new;
  int64_t vn_tok, vn_head;
  const int32_t* block_table;
  int64_t bt_row;
  const int32_t* seq_lens;
  const float* kd;
  int64_t kd_seq, kd_head;
  const float* vd;
  int64_t vd_seq, vd_head;
  uint8_t* k;
  int64_t k_page, k_row, k_head;  // bytes
  uint8_t* v;
  int64_t v_page, v_row, v_head;
  int num_seqs, n_new, h_k, d, page_shift, num_pages, max_blocks;
};

// (page, row) of new token t of sequence b, or page -1 when the sequence is
// shorter than n_new or its block-table entry lies outside the pool
__device__ __forceinline__ void new_token_slot(const int32_t* bt, int64_t bt_row, const int32_t* seq_lens, int b, int t,
                                               int n_new, int page_shift, int num_pages, int max_blocks, int& page,
                                               int& row) {
  const int pos = seq_lens[b] - n_new + t;
  page = -1;
  row = 0;
  if (pos < 0 || (pos >> page_shift) >= max_blocks) return;
  const int pg = bt[(int64_t)b * bt_row + (pos >> page_shift)];
  if (pg < 0 || pg >= num_pages) return;
  page = pg;
  row = pos & ((1 << page_shift) - 1);
}

__global__ __launch_bounds__(256) void write_kv_e4m3_kernel(WriteKvParams p) {
  // rows: (kv side s, token, head); 16 lanes cover up to 128 values of a row
  const int64_t rows = (int64_t)2 * p.num_seqs * p.n_new * p.h_k;
  const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int lane = threadIdx.x & 15;
  if (r >= rows) return;
  const int s = (int)(r / ((int64_t)p.num_seqs * p.n_new * p.h_k));
  const int64_t rem = r - (int64_t)s * p.num_seqs * p.n_new * p.h_k;
  const int tok = (int)(rem / p.h_k);
  const int g = (int)(rem - (int64_t)tok * p.h_k);
  const int b = tok / p.n_new, t = tok - b * p.n_new;
  int page, row;
  new_token_slot(p.block_table, p.bt_row, p.seq_lens, b, t, p.n_new, p.page_shift, p.num_pages, p.max_blocks, page,
                 row);
  if (page < 0) return;
  const uint8_t* src = s ? p.v_new + (int64_t)tok * p.vn_tok + (int64_t)g * p.vn_head
                         : p.k_new + (int64_t)tok * p.kn_tok + (int64_t)g * p.kn_head;
  const float descale = s ? p.vd[b * p.vd_seq + g * p.vd_head] : p.kd[b * p.kd_seq + g * p.kd_head];
  uint8_t* dst = s ? p.v + (int64_t)page * p.v_page + (int64_t)row * p.v_row + (int64_t)g * p.v_head
                   : p.k + (int64_t)page * p.k_page + (int64_t)row * p.k_row + (int64_t)g * p.k_head;
  for (int off = 8 * lane; off < p.d; off += 128) {
    float x[8];
    unpack8(*reinterpret_cast<const uint4*>(src + 2 * off), x);
    for (int e = 0; e < 8; ++e) x[e] = x[e] / descale;
    *reinterpret_cast<uint2*>(dst + off) = encode8(x);
  }
}

// ---- latent-record write: one wave per new token ----------------------------
// lane l: latent values 8l .. 8l+7 (block l / 16); lanes 0..7 copy the rope
struct WriteLatParams {
  const uint8_t* x_new;  // bf16 [tokens][576]
  int64_t xn_tok;        // bytes
  const int32_t* block_table;
  int64_t bt_row;
  const int32_t* seq_lens;
  uint8_t* lat;
  int64_t lat_page, lat_row;  // bytes
  uint8_t* rope;
  int64_t rope_page, rope_row;  // bytes
  uint8_t* scl;
  int64_t scl_page, scl_row;  // bytes
  int num_seqs, n_new, page_shift, num_pages, max_blocks;
};

__global__ __launch_bounds__(256) void write_kv_latent_kernel(WriteLatParams p) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= p.num_seqs * p.n_new) return;
  const int b = tok / p.n_new, t = tok - b * p.n_new;
  int page, row;
  new_token_slot(p.block_table, p.bt_row, p.seq_lens, b, t, p.n_new, p.page_shift, p.num_pages, p.max_blocks, page,
                 row);
  if (page < 0) return;  // wave-uniform
  const uint8_t* src = p.x_new + (int64_t)tok * p.xn_tok;
  float x[8];
  unpack8(*reinterpret_cast<const uint4*>(src + 2 * (8 * lane)), x);
  float m = 0.f;
  for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
  for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));  // 16 lanes = one 128-value block
  // the smallest power of two >= max(amax, 1e-6) / 448: adding an all-ones
  // mantissa carries into the exponent unless the mantissa is already zero
  const float scale = __uint_as_float((__float_as_uint(fmaxf(m, kMinAmax) / kE4m3Max) + 0x007FFFFFu) & 0xFF800000u);
  for (int e = 0; e < 8; ++e) x[e] = x[e] / scale;
  *reinterpret_cast<uint2*>(p.lat + (int64_t)page * p.lat_page + (int64_t)row * p.lat_row + 8 * lane) = encode8(x);
  if ((lane & 15) == 0)
    *reinterpret_cast<float*>(p.scl + (int64_t)page * p.scl_page + (int64_t)row * p.scl_row + 4 * (lane >> 4)) = scale;
  if (lane < 8)
    *reinterpret_cast<uint4*>(p.rope + (int64_t)page * p.rope_page + (int64_t)row * p.rope_row + 16 * lane) =
        *reinterpret_cast<const uint4*>(src + 2 * 512 + 16 * lane);
}

int log2_exact(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

}  // namespace

hipError_t quantize_q_launch(const pkv_quant_q_args& a, hipStream_t stream) {
  QuantQParams p;
  p.q = static_cast<const uint8_t*>(a.q);
  p.q_tok = a.q_tok_stride * 2;
  p.q_head = a.q_head_stride * 2;
  p.q8 = a.q8;
  p.q8_tok = a.q8_tok_stride;
  p.q8_head = a.q8_head_stride;
  p.qd = a.q_descale;
  p.qd_seq = a.qd_seq_stride;
  p.qd_head = a.qd_head_stride;
  p.q_len = a.q_len;
  p.h_r = a.h_q / a.h_k;
  p.d = a.d;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&quantize_q_kernel), dim3(a.num_seqs, a.h_k), dim3(256), args,
                         0, stream);
}

hipError_t write_kv_launch(const pkv_kv_write_args& a, hipStream_t stream) {
  if (a.kv_format == PKV_KV_MLA) {
    WriteLatParams p;
    p.x_new = static_cast<const uint8_t*>(a.k_new);
    p.xn_tok = a.kn_tok_stride * 2;
    p.block_table = a.block_table;
    p.bt_row = a.bt_row_stride;
    p.seq_lens = a.seq_lens;
    p.lat = a.k;
    p.lat_page = a.k_page_stride;
    p.lat_row = a.k_row_stride;
    p.rope = reinterpret_cast<uint8_t*>(a.k_rope);
    p.rope_page = a.rope_page_stride * 2;
    p.rope_row = a.rope_row_stride * 2;
    p.scl = reinterpret_cast<uint8_t*>(a.k_blk_scale);
    p.scl_page = a.scale_page_stride * 4;
    p.scl_row = a.scale_row_stride * 4;
    p.num_seqs = a.num_seqs;
    p.n_new = a.n_new;
    p.page_shift = log2_exact(a.page_size);
    p.num_pages = a.num_pages;
    p.max_blocks = a.max_blocks;
    const int tokens = a.num_seqs * a.n_new;
    void* args[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void*>(&write_kv_latent_kernel), dim3((tokens + 3) / 4), dim3(256),
                           args, 0, stream);
  }
  WriteKvParams p;
  p.k_new = static_cast<const uint8_t*>(a.k_new);
  p.kn_tok = a.kn_tok_stride * 2;
  p.kn_head = a.kn_head_stride * 2;
  p.v_new = static_cast<const uint8_t*>(a.v_new);
  p.vn_tok = a.vn_tok_stride * 2;
  p.vn_head = a.vn_head_stride * 2;
  p.block_table = a.block_table;
  p.bt_row = a.bt_row_stride;
  p.seq_lens = a.seq_lens;
  p.kd = a.k_descale;
  p.kd_seq = a.kd_seq_stride;
  p.kd_head = a.kd_head_stride;
  p.vd = a.v_descale;
  p.vd_seq = a.vd_seq_stride;
  p.vd_head = a.vd_head_stride;
  p.k = a.k;
  p.k_page = a.k_page_stride;
  p.k_row = a.k_row_stride;
  p.k_head = a.k_head_stride;
  p.v = a.v;
  p.v_page = a.v_page_stride;
  p.v_row = a.v_row_stride;
  p.v_head = a.v_head_stride;
  p.num_seqs = a.num_seqs;
  p.n_new = a.n_new;
  p.h_k = a.h_k;
  p.d = a.d;
  p.page_shift = log2_exact(a.page_size);
  p.num_pages = a.num_pages;
  p.max_blocks = a.max_blocks;
  const int64_t rows = (int64_t)2 * a.num_seqs * a.n_new * a.h_k;
  void* args[] = {&p};
  return hipLaunchKernel(reinterpret_cast<const void*>(&write_kv_e4m3_kernel), dim3((unsigned)((rows + 15) / 16)),
                         dim3(256), args, 0, stream);
}

}  // namespace pkv
