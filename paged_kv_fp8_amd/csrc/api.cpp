// Host entry points of libpkvfp8.so: argument validation and dispatch to
// the kernel launchers. Every check runs before any HIP call, so an invalid
// request returns its error code without touching the GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <unordered_map>

#include "pkv_internal.h"
#include "stamps.h"

namespace pkv {

namespace {
thread_local char g_last_error[512] = "";
}

pkv_status fail(pkv_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
bool pow2_page(int ps) { return ps == 16 || ps == 32 || ps == 64 || ps == 128; }

// Shape and mode checks shared by the slot query, the decode and the merge.
pkv_status check_shapes(const pkv_decode_args* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 1 || a->q_len < 1 || a->h_q < 1 || a->h_k < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs=%d q_len=%d h_q=%d h_k=%d must be >= 1", a->num_seqs, a->q_len,
                a->h_q, a->h_k);
  if (a->h_q % a->h_k) return fail(PKV_ERR_INVALID_ARG, "h_q=%d is not a multiple of h_k=%d", a->h_q, a->h_k);
  if (a->num_pages < 1 || a->max_blocks < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_pages=%d max_blocks=%d must be >= 1", a->num_pages, a->max_blocks);
  if (!pow2_page(a->page_size)) return fail(PKV_ERR_UNSUPPORTED, "page_size=%d not in {16,32,64,128}", a->page_size);
  if ((int64_t)a->max_blocks * a->page_size > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks * page_size exceeds int32");
  if (a->q_format != PKV_Q_BF16 && a->q_format != PKV_Q_E4M3)
    return fail(PKV_ERR_INVALID_ARG, "q_format=%d unknown", a->q_format);
  if (a->max_splits < 1 || a->max_splits > PKV_MAX_SPLITS)
    return fail(PKV_ERR_INVALID_ARG, "max_splits=%d not in [1, %d]", a->max_splits, PKV_MAX_SPLITS);
  if (!std::isfinite(a->softmax_scale) || !std::isfinite(a->o_scale))
    return fail(PKV_ERR_INVALID_ARG, "softmax_scale and o_scale must be finite");
  const int64_t rows = (int64_t)a->q_len * (a->h_q / a->h_k);
  if (a->kv_format == PKV_KV_E4M3) {
    if (a->d_qk != 128 || a->d_v != 128)
      return fail(PKV_ERR_UNSUPPORTED, "e4m3 cache: d_qk=%d d_v=%d, only 128/128 is built", a->d_qk, a->d_v);
    if (rows > 4096) return fail(PKV_ERR_UNSUPPORTED, "q_len * h_r = %lld rows > 4096", (long long)rows);
  } else if (narrow_kv(a->kv_format)) {
    if (a->d_qk != 128 || a->d_v != 128)
      return fail(PKV_ERR_UNSUPPORTED, "fp4/fp6 cache: d_qk=%d d_v=%d, only 128/128 is built", a->d_qk, a->d_v);
    if (a->q_format != PKV_Q_E4M3) return fail(PKV_ERR_UNSUPPORTED, "fp4/fp6 cache: the query must be e4m3");
    if (rows > 4096) return fail(PKV_ERR_UNSUPPORTED, "q_len * h_r = %lld rows > 4096", (long long)rows);
  } else if (a->kv_format == PKV_KV_MLA) {
    if (a->d_qk != 576 || a->d_v != 512 || a->h_k != 1)
      return fail(PKV_ERR_UNSUPPORTED, "latent cache needs h_k=1, d_qk=576, d_v=512 (got %d, %d, %d)", a->h_k,
                  a->d_qk, a->d_v);
    if (a->q_format != PKV_Q_BF16) return fail(PKV_ERR_UNSUPPORTED, "latent cache: only bf16 q is built");
    if (rows > 256) return fail(PKV_ERR_UNSUPPORTED, "latent cache: q_len * h_q = %lld rows > 256", (long long)rows);
  } else {
    return fail(PKV_ERR_INVALID_ARG, "kv_format=%d unknown", a->kv_format);
  }
  return PKV_OK;
}

bool bad_stride(int64_t s, int64_t elem_bytes, int64_t multiple) {
  return s < 0 || ((s * elem_bytes) % multiple) != 0;
}

pkv_status check_pointers(const pkv_decode_args* a, bool for_merge) {
  const bool mla = a->kv_format == PKV_KV_MLA;
  const int64_t q_elem = a->q_format == PKV_Q_BF16 ? 2 : 1;
  const int64_t q_mult = a->q_format == PKV_Q_BF16 ? 16 : 8;
  if (!a->o || !a->lse || !a->seq_lens || !a->n_splits)
    return fail(PKV_ERR_INVALID_ARG, "o, lse, seq_lens and n_splits must be non-NULL");
  if (!aligned(a->o, 16) || !aligned(a->lse, 4) || bad_stride(a->o_tok_stride, 2, 16) ||
      bad_stride(a->o_head_stride, 2, 16))
    return fail(PKV_ERR_INVALID_ARG, "o must be 16-B aligned with 16-B multiple strides");
  if (a->max_splits > 1) {
    const size_t need = pkv_workspace_bytes(a->num_seqs, a->h_k, a->q_len * (a->h_q / a->h_k), a->d_v, a->max_splits);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for max_splits=%d", a->workspace_bytes, need,
                  a->max_splits);
    if (!aligned(a->workspace, 16)) return fail(PKV_ERR_INVALID_ARG, "workspace must be 16-B aligned");
  }
  if (for_merge) return PKV_OK;
  if (!a->q || !a->k || !a->block_table || !a->work)
    return fail(PKV_ERR_INVALID_ARG, "q, k, block_table and work must be non-NULL");
  if (a->num_work < 1) return fail(PKV_ERR_INVALID_ARG, "num_work=%d < 1", a->num_work);
  if (!aligned(a->q, 16) || bad_stride(a->q_tok_stride, q_elem, q_mult) || bad_stride(a->q_head_stride, q_elem, q_mult))
    return fail(PKV_ERR_INVALID_ARG, "q must be 16-B aligned with %lld-B multiple strides", (long long)q_mult);
  if (!aligned(a->work, 16)) return fail(PKV_ERR_INVALID_ARG, "work must be 16-B aligned");
  if (a->bin_offsets && (a->num_bins < 1 || !aligned(a->bin_offsets, 4)))
    return fail(PKV_ERR_INVALID_ARG, "bin_offsets needs num_bins >= 1 and 4-B alignment");
  if (narrow_kv(a->kv_format) && (a->bin_offsets || a->queue))
    return fail(PKV_ERR_UNSUPPORTED, "fp4/fp6 cache: only the one-wave plan (pkv_plan_split_kv) is built");
  if (a->work_in_keys != 0 && a->work_in_keys != 1)
    return fail(PKV_ERR_INVALID_ARG, "work_in_keys=%d must be 0 or 1", a->work_in_keys);
  if (a->work_in_keys && mla) return fail(PKV_ERR_UNSUPPORTED, "latent cache: plans in 128-key tiles only");
  if (a->work_pairs != 0 && a->work_pairs != 1)
    return fail(PKV_ERR_INVALID_ARG, "work_pairs=%d must be 0 or 1", a->work_pairs);
  if (a->work_pairs) {
    if (mla || a->h_k != 4 || a->q_len * (a->h_q / a->h_k) > 16)
      return fail(PKV_ERR_UNSUPPORTED, "work_pairs: built for four kv heads of at most 16 rows (h_k=%d, rows=%d)",
                  a->h_k, a->q_len * (a->h_q / a->h_k));
    if (a->bin_offsets || a->queue || a->work_in_keys)
      return fail(PKV_ERR_INVALID_ARG, "work_pairs: a pkv_plan_paired plan (no bins, queue or key ranges)");
    if (a->num_work % 2) return fail(PKV_ERR_INVALID_ARG, "work_pairs: num_work=%d must be even", a->num_work);
  }
  if (a->kv_format == PKV_KV_NVFP4) {
    if (!a->k_group_scale || !a->v_group_scale)
      return fail(PKV_ERR_INVALID_ARG, "NVFP4 cache: k_group_scale and v_group_scale must be non-NULL");
    if (!aligned(a->k_group_scale, 8) || bad_stride(a->kgs_page_stride, 1, 8) || bad_stride(a->kgs_row_stride, 1, 8) ||
        bad_stride(a->kgs_head_stride, 1, 8))
      return fail(PKV_ERR_INVALID_ARG, "k_group_scale must be 8-B aligned with 8-B multiple strides");
    if (a->vgs_page_stride < 0 || a->vgs_row_stride < 0 || a->vgs_head_stride < 0)
      return fail(PKV_ERR_INVALID_ARG, "v_group_scale strides must be >= 0");
  }
  if (a->queue) {
    if (!a->bin_offsets) return fail(PKV_ERR_INVALID_ARG, "queue needs bin_offsets (a plan from pkv_plan_queued)");
    if (!aligned(a->queue, 4)) return fail(PKV_ERR_INVALID_ARG, "queue must be 4-B aligned");
    if (mla) return fail(PKV_ERR_UNSUPPORTED, "latent cache: the queued plan is built for the e4m3 cache only");
  }
  if (a->bt_row_stride < a->max_blocks)
    return fail(PKV_ERR_INVALID_ARG, "bt_row_stride=%lld < max_blocks=%d", (long long)a->bt_row_stride,
                a->max_blocks);
  if (!aligned(a->k, 16) || bad_stride(a->k_page_stride, 1, 16) || bad_stride(a->k_row_stride, 1, 16) ||
      bad_stride(a->k_head_stride, 1, 16))
    return fail(PKV_ERR_INVALID_ARG, "k must be 16-B aligned with 16-B multiple strides");
  if (mla) {
    if (a->v && a->v != a->k) return fail(PKV_ERR_INVALID_ARG, "latent cache: v must be NULL or equal k");
    if (!a->k_rope || !a->k_blk_scale) return fail(PKV_ERR_INVALID_ARG, "latent cache: k_rope, k_blk_scale NULL");
    if (!aligned(a->k_rope, 16) || bad_stride(a->rope_page_stride, 2, 16) || bad_stride(a->rope_row_stride, 2, 16))
      return fail(PKV_ERR_INVALID_ARG, "k_rope must be 16-B aligned with 16-B multiple strides");
    if (!aligned(a->k_blk_scale, 16) || bad_stride(a->scale_page_stride, 4, 16) ||
        bad_stride(a->scale_row_stride, 4, 16))
      return fail(PKV_ERR_INVALID_ARG, "k_blk_scale must be 16-B aligned with 16-B multiple strides");
    if ((int64_t)a->page_size * a->k_row_stride >= (int64_t)1 << 30 ||
        (int64_t)a->page_size * a->rope_row_stride * 2 >= (int64_t)1 << 30 ||
        (int64_t)a->page_size * a->scale_row_stride * 4 >= (int64_t)1 << 30)
      return fail(PKV_ERR_UNSUPPORTED, "latent cache: page_size * row stride must be below 2^30 bytes");
    return PKV_OK;
  }
  if (!a->v || !aligned(a->v, 16) || bad_stride(a->v_page_stride, 1, 16) || bad_stride(a->v_row_stride, 1, 16) ||
      bad_stride(a->v_head_stride, 1, 16))
    return fail(PKV_ERR_INVALID_ARG, "v must be non-NULL, 16-B aligned, with 16-B multiple strides");
  if ((int64_t)a->page_size * a->k_row_stride >= (int64_t)1 << 30 ||
      (int64_t)a->page_size * a->v_row_stride >= (int64_t)1 << 30)
    return fail(PKV_ERR_UNSUPPORTED, "page_size * k/v row stride must be below 2^30 bytes");
  if (a->k_page_stride >= (int64_t)1 << 32 || a->v_page_stride >= (int64_t)1 << 32 ||
      (a->kv_format == PKV_KV_NVFP4 && (a->kgs_page_stride >= (int64_t)1 << 32 || a->vgs_page_stride >= (int64_t)1 << 32)))
    return fail(PKV_ERR_UNSUPPORTED, "page strides must be below 2^32 bytes");
  if (!a->k_descale || !a->v_descale || (a->q_format == PKV_Q_E4M3 && !a->q_descale))
    return fail(PKV_ERR_INVALID_ARG, "k/v descale (and q descale for e4m3 q) must be non-NULL");
  if (a->kd_seq_stride < 0 || a->kd_head_stride < 0 || a->vd_seq_stride < 0 || a->vd_head_stride < 0 ||
      a->qd_seq_stride < 0 || a->qd_head_stride < 0)
    return fail(PKV_ERR_INVALID_ARG, "descale strides must be >= 0");
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

hipError_t check_lds(const void* kernel, size_t dyn_lds) {
  // static LDS per kernel, looked up once
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> static_bytes;
  size_t fixed = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = static_bytes.find(kernel);
    if (it == static_bytes.end()) {
      hipFuncAttributes attr;
      const hipError_t e = hipFuncGetAttributes(&attr, kernel);
      if (e != hipSuccess) return e;
      it = static_bytes.emplace(kernel, attr.sharedSizeBytes).first;
    }
    fixed = it->second;
  }
  return fixed + dyn_lds <= kMaxLdsBytes ? hipSuccess : hipErrorInvalidConfiguration;
}
}  // namespace pkv

using namespace pkv;

extern "C" const char* pkv_status_string(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_CAPACITY: return "PKV_ERR_CAPACITY";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    default: return "PKV_ERR_UNKNOWN";
  }
}

extern "C" const char* pkv_last_error(void) { return g_last_error; }

extern "C" int32_t pkv_version(void) { return 100; }

extern "C" size_t pkv_decode_args_size(void) { return sizeof(pkv_decode_args); }

extern "C" size_t pkv_workspace_bytes(int32_t num_seqs, int32_t h_k, int32_t n_rows, int32_t d_v, int32_t max_splits) {
  if (num_seqs < 1 || h_k < 1 || n_rows < 1 || d_v < 1 || max_splits < 1) return 0;
  const size_t floats = (size_t)max_splits * num_seqs * h_k * n_rows * ((size_t)d_v + 2);
  return (floats * 4 + 255) / 256 * 256;
}

extern "C" pkv_status pkv_decode_slots(const pkv_decode_args* a, int32_t* cu_count, int32_t* wg_per_cu,
                                       int32_t* n_q_tiles) {
  pkv_status st = check_shapes(a);
  if (st != PKV_OK) return st;
  if (!cu_count || !wg_per_cu || !n_q_tiles) return fail(PKV_ERR_INVALID_ARG, "slot outputs must be non-NULL");
  int dev = 0, cus = 0, wgs = 0;
  if ((st = hip_status(hipGetDevice(&dev), "hipGetDevice")) != PKV_OK) return st;
  if ((st = hip_status(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev), "CU count")) != PKV_OK)
    return st;
  const int64_t rows = (int64_t)a->q_len * (a->h_q / a->h_k);
  int per_tile;
  if (a->kv_format == PKV_KV_MLA) {
    per_tile = mla_rows_per_tile(*a);
    st = hip_status(mla_occupancy(*a, &wgs), "occupancy");
  } else {
    const GqaVariant v = gqa_variant(*a);
    per_tile = gqa_rows_per_tile(v);
    st = hip_status(gqa_occupancy(v, &wgs), "occupancy");
  }
  if (st != PKV_OK) return st;
  *cu_count = cus;
  *wg_per_cu = wgs < 1 ? 1 : wgs;
  *n_q_tiles = (int32_t)((rows + per_tile - 1) / per_tile);
  return PKV_OK;
}

extern "C" const char* pkv_decode_kernel_name(const pkv_decode_args* a) {
  if (check_shapes(a) != PKV_OK) return nullptr;
  return a->kv_format == PKV_KV_MLA ? mla_kernel_name(*a) : "gqa_decode_kernel";
}

extern "C" pkv_status pkv_paged_decode_attn(const pkv_decode_args* a, void* stream) {
  pkv_status st = check_shapes(a);
  if (st != PKV_OK) return st;
  if ((st = check_pointers(a, false)) != PKV_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->kv_format == PKV_KV_MLA) return hip_status(mla_launch(*a, s), "latent decode launch");
  return hip_status(gqa_launch(*a, gqa_variant(*a), s), "decode launch");
}

extern "C" pkv_status pkv_merge_splits(const pkv_decode_args* a, void* stream) {
  pkv_status st = check_shapes(a);
  if (st != PKV_OK) return st;
  if ((st = check_pointers(a, true)) != PKV_OK) return st;
  if (a->max_splits == 1) return PKV_OK;
  return hip_status(merge_launch(*a, static_cast<hipStream_t>(stream)), "merge launch");
}

// ---- decode step without allocation ------------------------------------------
// The split workspace of pkv_paged_decode_noalloc: a module-scope device array,
// so each device the library runs on holds one copy from the first call until
// the process ends. Host code never uses its name as an address: the address
// on the current device comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

pkv_status scratch_on_current_device(void** out) {
  int dev = 0;
  pkv_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != PKV_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((st = hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) != PKV_OK)
      return st;
    if (!ptr) return fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}
}  // namespace

extern "C" pkv_status pkv_paged_decode_noalloc(const pkv_decode_args* a, void* stream) {
  pkv_status st = check_shapes(a);
  if (st != PKV_OK) return st;
  if (a->queue) return fail(PKV_ERR_UNSUPPORTED, "no-allocation decode: the queued plan is not taken");
  const size_t need = a->max_splits > 1 ? pkv_workspace_bytes(a->num_seqs, a->h_k, a->q_len * (a->h_q / a->h_k),
                                                               a->d_v, a->max_splits)
                                        : 0;
  if (need > (size_t)PKV_NOALLOC_WORKSPACE_BYTES)
    return fail(PKV_ERR_WORKSPACE, "no-allocation decode: %zu bytes of split workspace needed, the library holds %zu",
                need, (size_t)PKV_NOALLOC_WORKSPACE_BYTES);
  pkv_decode_args b = *a;
  // validate everything else with a stand-in workspace before any HIP call
  b.workspace = reinterpret_cast<void*>(uintptr_t{256});
  b.workspace_bytes = PKV_NOALLOC_WORKSPACE_BYTES;
  if ((st = check_pointers(&b, false)) != PKV_OK) return st;
  if (need > 0) {
    if ((st = scratch_on_current_device(&b.workspace)) != PKV_OK) return st;
  } else {
    b.workspace = nullptr;
    b.workspace_bytes = 0;
  }
  if ((st = pkv_paged_decode_attn(&b, stream)) != PKV_OK) return st;
  return pkv_merge_splits(&b, stream);
}

namespace {
bool bad_elem_stride(int64_t s, int64_t mult) { return s < 0 || s % mult != 0; }
}  // namespace

extern "C" pkv_status pkv_quantize_q(const pkv_quant_q_args* a, void* stream) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 1 || a->q_len < 1 || a->h_q < 1 || a->h_k < 1 || a->d < 8)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs=%d q_len=%d h_q=%d h_k=%d d=%d: sizes must be >= 1 (d >= 8)", a->num_seqs,
                a->q_len, a->h_q, a->h_k, a->d);
  if (a->h_q % a->h_k) return fail(PKV_ERR_INVALID_ARG, "h_q=%d is not a multiple of h_k=%d", a->h_q, a->h_k);
  if (a->d % 8) return fail(PKV_ERR_INVALID_ARG, "d=%d is not a multiple of 8", a->d);
  if (!a->q || !a->q8 || !a->q_descale) return fail(PKV_ERR_INVALID_ARG, "q, q8 and q_descale must be non-NULL");
  if (!aligned(a->q, 16) || bad_elem_stride(a->q_tok_stride, 8) || bad_elem_stride(a->q_head_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "q must be 16-B aligned with strides that are multiples of 8 elements");
  if (!aligned(a->q8, 8) || bad_elem_stride(a->q8_tok_stride, 8) || bad_elem_stride(a->q8_head_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "q8 must be 8-B aligned with strides that are multiples of 8 bytes");
  if (!aligned(a->q_descale, 4) || a->qd_seq_stride < 0 || a->qd_head_stride < 0)
    return fail(PKV_ERR_INVALID_ARG, "q_descale must be 4-B aligned with strides >= 0");
  return hip_status(quantize_q_launch(*a, static_cast<hipStream_t>(stream)), "query quantisation launch");
}

extern "C" pkv_status pkv_write_kv(const pkv_kv_write_args* a, void* stream) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 1 || a->n_new < 1 || a->h_k < 1 || a->d < 8 || a->num_pages < 1 || a->max_blocks < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs, n_new, h_k, num_pages, max_blocks must be >= 1 and d >= 8");
  if (!pow2_page(a->page_size)) return fail(PKV_ERR_UNSUPPORTED, "page_size=%d not in {16,32,64,128}", a->page_size);
  if (!a->k_new || !a->block_table || !a->seq_lens || !a->k)
    return fail(PKV_ERR_INVALID_ARG, "k_new, block_table, seq_lens and k must be non-NULL");
  if (a->bt_row_stride < a->max_blocks) return fail(PKV_ERR_INVALID_ARG, "bt_row_stride < max_blocks");
  if (!aligned(a->k_new, 16) || bad_elem_stride(a->kn_tok_stride, 8) || bad_elem_stride(a->kn_head_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "k_new must be 16-B aligned with strides that are multiples of 8 elements");
  if (!aligned(a->k, 8) || bad_elem_stride(a->k_page_stride, 8) || bad_elem_stride(a->k_row_stride, 8) ||
      bad_elem_stride(a->k_head_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "k must be 8-B aligned with strides that are multiples of 8 bytes");
  if (a->kv_format == PKV_KV_MLA) {
    if (a->h_k != 1 || a->d != 576) return fail(PKV_ERR_INVALID_ARG, "latent write needs h_k = 1 and d = 576");
    if (!a->k_rope || !a->k_blk_scale) return fail(PKV_ERR_INVALID_ARG, "latent write: k_rope, k_blk_scale NULL");
    if (!aligned(a->k_rope, 16) || bad_elem_stride(a->rope_page_stride, 8) || bad_elem_stride(a->rope_row_stride, 8))
      return fail(PKV_ERR_INVALID_ARG, "k_rope must be 16-B aligned with strides that are multiples of 8 elements");
    if (!aligned(a->k_blk_scale, 4) || a->scale_page_stride < 0 || a->scale_row_stride < 0)
      return fail(PKV_ERR_INVALID_ARG, "k_blk_scale must be 4-B aligned with strides >= 0");
  } else if (a->kv_format == PKV_KV_E4M3) {
    if (a->d % 8) return fail(PKV_ERR_INVALID_ARG, "d=%d is not a multiple of 8", a->d);
    if (!a->v_new || !a->v || !a->k_descale || !a->v_descale)
      return fail(PKV_ERR_INVALID_ARG, "v_new, v, k_descale and v_descale must be non-NULL");
    if (!aligned(a->v_new, 16) || bad_elem_stride(a->vn_tok_stride, 8) || bad_elem_stride(a->vn_head_stride, 8))
      return fail(PKV_ERR_INVALID_ARG, "v_new must be 16-B aligned with strides that are multiples of 8 elements");
    if (!aligned(a->v, 8) || bad_elem_stride(a->v_page_stride, 8) || bad_elem_stride(a->v_row_stride, 8) ||
        bad_elem_stride(a->v_head_stride, 8))
      return fail(PKV_ERR_INVALID_ARG, "v must be 8-B aligned with strides that are multiples of 8 bytes");
    if (a->kd_seq_stride < 0 || a->kd_head_stride < 0 || a->vd_seq_stride < 0 || a->vd_head_stride < 0)
      return fail(PKV_ERR_INVALID_ARG, "descale strides must be >= 0");
  } else {
    return fail(PKV_ERR_UNSUPPORTED, "kv_format=%d", a->kv_format);
  }
  return hip_status(write_kv_launch(*a, static_cast<hipStream_t>(stream)), "KV-cache write launch");
}

extern "C" size_t pkv_quant_q_args_size(void) { return sizeof(pkv_quant_q_args); }

extern "C" size_t pkv_kv_write_args_size(void) { return sizeof(pkv_kv_write_args); }

namespace {
// Checks of one slot list of a sparse decode call (nothing is read when the
// list is unused).
pkv_status check_sparse_list(const pkv_sparse_list& l, int idx) {
  if (l.width < 0) return fail(PKV_ERR_INVALID_ARG, "list[%d].width=%d < 0", idx, l.width);
  if (l.width == 0) return PKV_OK;
  if (l.width > 4096) return fail(PKV_ERR_UNSUPPORTED, "list[%d].width=%d > 4096", idx, l.width);
  if (!pow2_page(l.page_size))
    return fail(PKV_ERR_UNSUPPORTED, "list[%d].page_size=%d not in {16,32,64,128}", idx, l.page_size);
  if (l.num_pages < 1 || (int64_t)l.num_pages * l.page_size >= (int64_t{1} << 31))
    return fail(PKV_ERR_INVALID_ARG, "list[%d].num_pages=%d: need 1 <= num_pages * page_size < 2^31", idx,
                l.num_pages);
  if (!l.latent || !l.rope || !l.blk_scale || !l.slots)
    return fail(PKV_ERR_INVALID_ARG, "list[%d]: latent, rope, blk_scale and slots must be non-NULL", idx);
  if (!aligned(l.latent, 16) || bad_elem_stride(l.lat_page_stride, 16) || bad_elem_stride(l.lat_row_stride, 16))
    return fail(PKV_ERR_INVALID_ARG, "list[%d].latent must be 16-B aligned with 16-B multiple strides", idx);
  if (!aligned(l.rope, 16) || bad_elem_stride(l.rope_page_stride, 8) || bad_elem_stride(l.rope_row_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "list[%d].rope must be 16-B aligned with strides of 8 elements", idx);
  if (!aligned(l.blk_scale, 8) || bad_elem_stride(l.scale_page_stride, 2) || bad_elem_stride(l.scale_row_stride, 2))
    return fail(PKV_ERR_INVALID_ARG, "list[%d].blk_scale must be 8-B aligned with even strides", idx);
  if (!aligned(l.slots, 4) || l.slots_row_stride < l.width)
    return fail(PKV_ERR_INVALID_ARG, "list[%d].slots must be 4-B aligned with row stride >= width", idx);
  return PKV_OK;
}

pkv_status check_sparse(const pkv_sparse_args* a) {
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->num_tokens < 1 || a->h_q < 1)
    return fail(PKV_ERR_INVALID_ARG, "num_tokens=%d h_q=%d must be >= 1", a->num_tokens, a->h_q);
  if (a->h_q % 16 || a->h_q > 128) return fail(PKV_ERR_UNSUPPORTED, "h_q=%d: a multiple of 16 up to 128", a->h_q);
  if (a->num_tokens > 65535) return fail(PKV_ERR_UNSUPPORTED, "num_tokens=%d > 65535", a->num_tokens);
  if (!std::isfinite(a->softmax_scale) || !std::isfinite(a->o_scale))
    return fail(PKV_ERR_INVALID_ARG, "softmax_scale and o_scale must be finite");
  if (!a->q || !a->o || !a->lse) return fail(PKV_ERR_INVALID_ARG, "q, o and lse must be non-NULL");
  if (!aligned(a->q, 16) || bad_elem_stride(a->q_tok_stride, 8) || bad_elem_stride(a->q_head_stride, 8))
    return fail(PKV_ERR_INVALID_ARG, "q must be 16-B aligned with strides that are multiples of 8 elements");
  if (!aligned(a->o, 8) || bad_elem_stride(a->o_tok_stride, 4) || bad_elem_stride(a->o_head_stride, 4))
    return fail(PKV_ERR_INVALID_ARG, "o must be 8-B aligned with strides that are multiples of 4 elements");
  if (!aligned(a->lse, 4)) return fail(PKV_ERR_INVALID_ARG, "lse must be 4-B aligned");
  if (a->sink && !aligned(a->sink, 4)) return fail(PKV_ERR_INVALID_ARG, "sink must be 4-B aligned");
  for (int i = 0; i < 2; ++i) {
    const pkv_status st = check_sparse_list(a->list[i], i);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}
}  // namespace

extern "C" int64_t pkv_sparse_workspace_bytes(const pkv_sparse_args* a) {
  if (check_sparse(a) != PKV_OK) return 0;
  return sparse_ws_bytes(*a);
}

namespace {
pkv_status sparse_call(const pkv_sparse_args* a, void* stream, bool tiles, bool merge) {
  pkv_status st = check_sparse(a);
  if (st != PKV_OK) return st;
  const int64_t need = sparse_ws_bytes(*a);
  if (need > 0 && (!a->workspace || !aligned(a->workspace, 256) || a->workspace_bytes < need))
    return fail(PKV_ERR_WORKSPACE, "workspace: %lld bytes needed, 256-B aligned (got %lld)", (long long)need,
                (long long)a->workspace_bytes);
  return hip_status(sparse_launch(*a, static_cast<hipStream_t>(stream), tiles, merge), "sparse decode launch");
}
}  // namespace

extern "C" pkv_status pkv_sparse_decode(const pkv_sparse_args* a, void* stream) {
  return sparse_call(a, stream, true, true);
}

extern "C" pkv_status pkv_sparse_tiles(const pkv_sparse_args* a, void* stream) {
  return sparse_call(a, stream, true, false);
}

extern "C" pkv_status pkv_sparse_merge(const pkv_sparse_args* a, void* stream) {
  return sparse_call(a, stream, false, true);
}

extern "C" size_t pkv_sparse_args_size(void) { return sizeof(pkv_sparse_args); }

extern "C" pkv_status pkv_debug_stamps(int32_t loop, uint64_t* host_dst) {
  if (!host_dst) return fail(PKV_ERR_INVALID_ARG, "host_dst must be non-NULL");
  if (loop != 0 && loop != 1) return fail(PKV_ERR_INVALID_ARG, "loop=%d must be 0 (kv-head) or 1 (latent)", loop);
#if PKV_STAMPS
  static_assert(PKV_STAMP_WORDS == kStampWords, "stamp layout");
  return hip_status(loop == 0 ? gqa_copy_stamps(host_dst) : mla_copy_stamps(host_dst), "stamps copy");
#else
  return fail(PKV_ERR_UNSUPPORTED, "library built without -DPKV_STAMPS=1");
#endif
}

extern "C" pkv_status pkv_stream_read_probe(const void* src, size_t bytes, int32_t workgroups, int32_t unroll,
                                            uint32_t* sink, void* stream) {
  if (!src || !sink) return fail(PKV_ERR_INVALID_ARG, "src and sink must be non-NULL");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(PKV_ERR_INVALID_ARG, "src must be 16-B aligned, sink 4-B");
  if (unroll != 4 && unroll != 8 && unroll != 16) return fail(PKV_ERR_INVALID_ARG, "unroll=%d not in {4, 8, 16}", unroll);
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "workgroups=%d not in [1, 2^20]", workgroups);
  const size_t chunk = (size_t)4096 * unroll;
  if (bytes == 0 || bytes % chunk) return fail(PKV_ERR_INVALID_ARG, "bytes=%zu not a positive multiple of %zu", bytes, chunk);
  return hip_status(probe_launch(src, bytes, workgroups, unroll, sink, static_cast<hipStream_t>(stream)),
                    "probe launch");
}
