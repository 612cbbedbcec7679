// Combine of split-KV partials ("mjolnir-kernel 0.1.0 wheel:
// mjolnir/t5_decode.py", reduction kernel and the module docstring's
// "Workspace" paragraph): per row of a split sequence, the partials of the
// splits it used are weighted by exp(m_j - max m) and normalised by the
// weighted sum of the l_j. Only the splits a sequence used are read, so the
// workspace needs no initialisation; sequences with one split were written
// by the decode and are skipped. The j order is fixed, so the result is
// deterministic.
//
// gfx950 layout: one thread owns 4 consecutive d_v values of one row (one
// 16-byte load per split, one 8-byte bf16 store), 256 threads per
// workgroup; the (max, sum) pairs of a row are read by all its threads from
// the same cache lines.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct MergeParams {
  const float* ws_o;
  const float2* ws_ml;
  const int32_t* n_splits;
  uint8_t* o;
  int64_t o_tok, o_head;  // bytes
  float* lse;
  int64_t total_rows;  // num_seqs * h_k * rows
  int64_t split_stride;  // rows between consecutive split slots (= total_rows)
  float o_scale;
  int h_k, rows, h_r, q_len, d_v, max_splits;
};

// kSplitsPerRound splits are read per round with independent loads, so a
// row of up to that many splits costs one memory latency.
constexpr int kSplitsPerRound = 16;

template <int DV>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int kThreadsPerRow = DV / 4;  // 4 d_v values (one 16-byte load) per thread
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  const int tr = threadIdx.x / kThreadsPerRow;
  const int tc = threadIdx.x % kThreadsPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + tr;
  if (row >= p.total_rows) return;
  const int b = (int)(row / ((int64_t)p.h_k * p.rows));
  const int rem = (int)(row - (int64_t)b * p.h_k * p.rows);
  const int g = rem / p.rows;
  const int n = rem - g * p.rows;
  int ns = p.n_splits[b];
  if (ns <= 1) return;  // written by the decode
  ns = min(ns, p.max_splits);

  // One round trip for up to kSplitsPerRound splits: the (max, sum) pairs and
  // the partial rows are independent loads, issued together. A longer split
  // list takes one round trip per round: each round's weights use the max so
  // far, and what was summed before is rescaled when a round raises it (with
  // one round, the sums are those of the plain weighted combine).
  float2 ml[kSplitsPerRound];
  f32x4 oj[kSplitsPerRound];
  float m_star = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int j0 = 0; j0 < ns; j0 += kSplitsPerRound) {
#pragma unroll
    for (int u = 0; u < kSplitsPerRound; ++u) {
      const bool ok = j0 + u < ns;
      const int64_t pr = (int64_t)(j0 + u) * p.split_stride + row;
      ml[u] = ok ? p.ws_ml[pr] : float2{-INFINITY, 0.f};
      oj[u] = ok ? *reinterpret_cast<const f32x4*>(p.ws_o + pr * DV + 4 * tc) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m_new = m_star;
#pragma unroll
    for (int u = 0; u < kSplitsPerRound; ++u) m_new = fmaxf(m_new, ml[u].x);
    if (m_new == -INFINITY) continue;  // no split of this row saw a key yet
    if (m_new != m_star) {
      const float sc = m_star == -INFINITY ? 0.f : __expf(m_star - m_new);
      acc *= sc;
      den *= sc;
      m_star = m_new;
    }
#pragma unroll
    for (int u = 0; u < kSplitsPerRound; ++u) {
      const float wgt = ml[u].x == -INFINITY ? 0.f : __expf(ml[u].x - m_star);
      den += wgt * ml[u].y;
      acc += wgt * oj[u];
    }
  }
  const float inv = den > 0.f ? p.o_scale / den : 0.f;
  const int qi = n / p.h_r;
  const int hr = n - qi * p.h_r;
  uint8_t* orow = p.o + (int64_t)(b * p.q_len + qi) * p.o_tok + (int64_t)(g * p.h_r + hr) * p.o_head;
  bf16x4 out;
  for (int e = 0; e < 4; ++e) out[e] = (__bf16)(acc[e] * inv);
  *reinterpret_cast<bf16x4*>(orow + 2 * (4 * tc)) = out;
  if (tc == 0) p.lse[row] = den > 0.f ? m_star + logf(den) : -INFINITY;
}

}  // namespace

hipError_t merge_launch(const pkv_decode_args& a, hipStream_t stream) {
  MergeParams p;
  const int64_t rows_all = ws_rows(a);
  p.ws_o = static_cast<const float*>(a.workspace);
  p.ws_ml = reinterpret_cast<const float2*>(p.ws_o + (int64_t)a.max_splits * rows_all * a.d_v);
  p.n_splits = a.n_splits;
  p.o = static_cast<uint8_t*>(a.o);
  p.o_tok = a.o_tok_stride * 2;
  p.o_head = a.o_head_stride * 2;
  p.lse = a.lse;
  p.total_rows = rows_all;
  p.split_stride = rows_all;
  p.o_scale = a.o_scale;
  p.h_k = a.h_k;
  p.h_r = a.h_q / a.h_k;
  p.q_len = a.q_len;
  p.rows = a.q_len * p.h_r;
  p.d_v = a.d_v;
  p.max_splits = a.max_splits;
  void* args[] = {&p};
  if (a.d_v == 128) {
    const int64_t blocks = (rows_all + 7) / 8;
    return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<128>), dim3((unsigned)blocks), dim3(256),
                           args, 0, stream);
  }
  const int64_t blocks = (rows_all + 1) / 2;
  return hipLaunchKernel(reinterpret_cast<const void*>(&merge_kernel<512>), dim3((unsigned)blocks), dim3(256), args,
                         0, stream);
}

}  // namespace pkv
