// Internal declarations shared by the host entry points and the kernel
// launchers of libpkvfp8.so. Not installed; the public ABI is pkv_fp8.h.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "pkv_fp8.h"

namespace pkv {

// Records a one-line reason for the calling thread's current failure and
// returns `code`, so call sites read `return fail(PKV_ERR_..., "...", ...)`.
pkv_status fail(pkv_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Kernel selection for the e4m3 K/V cache (d = 128) family.
struct GqaVariant {
  bool fp8_q;       // e4m3 Q, e4m3 P, fp8 MFMA; else bf16 Q, bf16 P, bf16 MFMA
  int n_blocks;     // 16-row N blocks per wave (1 or 2)
  bool causal_tail; // q_len > 1 && causal
  int stages;       // register ring depth of the KV stream (blocks of 32 keys)
  int heads_per_wg; // kv heads (one wave each) per workgroup
  bool stream;      // balanced plan: each workgroup streams the items of its bin
  int kvf;          // K/V format: 0 = e4m3, else the packed narrow format's PKV_KV_* value (one-item form only)
  bool paired;      // paired plan: two work items per workgroup, one wave per (item, kv head)
};

// Packed narrow K/V formats (fp4 e2m1, fp6 e2m3 / e3m2).
inline bool narrow_kv(int kv_format) {
  return kv_format == PKV_KV_E2M1 || kv_format == PKV_KV_E2M3 || kv_format == PKV_KV_E3M2 ||
         kv_format == PKV_KV_NVFP4;
}
// LDS of one CU, the most one workgroup may hold (static + dynamic bytes).
constexpr size_t kMaxLdsBytes = 160 * 1024;
// hipSuccess when `kernel` launched with `dyn_lds` bytes of dynamic LDS fits
// kMaxLdsBytes, else hipErrorInvalidConfiguration (nothing is launched):
// the command processor rejects a dispatch that asks for more, and that
// aborts the whole queue rather than failing the launch.
hipError_t check_lds(const void* kernel, size_t dyn_lds);

GqaVariant gqa_variant(const pkv_decode_args& a);
int gqa_rows_per_tile(const GqaVariant& v);
hipError_t gqa_occupancy(const GqaVariant& v, int* units_per_cu);
hipError_t gqa_launch(const pkv_decode_args& a, const GqaVariant& v, hipStream_t stream);

// Latent-record (MLA) family.
int mla_rows_per_tile(const pkv_decode_args& a);
const char* mla_kernel_name(const pkv_decode_args& a);  // "mla_pair_kernel" or "mla_lds_kernel"
hipError_t mla_occupancy(const pkv_decode_args& a, int* wg_per_cu);
hipError_t mla_launch(const pkv_decode_args& a, hipStream_t stream);

// Sparse slot-list decode over latent records (tile kernel + merge).
int sparse_tiles(const pkv_sparse_args& a);
int64_t sparse_ws_bytes(const pkv_sparse_args& a);
hipError_t sparse_launch(const pkv_sparse_args& a, hipStream_t stream, bool tiles, bool merge);

// Combine of split partials.
hipError_t merge_launch(const pkv_decode_args& a, hipStream_t stream);
hipError_t quantize_q_launch(const pkv_quant_q_args& a, hipStream_t stream);
hipError_t write_kv_launch(const pkv_kv_write_args& a, hipStream_t stream);

// Stamps of the one-item kv-head loop / the latent staged loop (library
// built with -DPKV_STAMPS=1; hipErrorNotSupported otherwise).
hipError_t gqa_copy_stamps(void* host_dst);
hipError_t mla_copy_stamps(void* host_dst);

// Streaming-read probe (measurement only).
hipError_t probe_launch(const void* src, size_t bytes, int workgroups, int unroll, uint32_t* sink,
                        hipStream_t stream);

// Workspace partition, in floats: partial O of every (split, seq, head,
// row) first, then its (max, sum) pair.
inline int64_t ws_rows(const pkv_decode_args& a) {
  return (int64_t)a.num_seqs * a.h_k * a.q_len * (a.h_q / a.h_k);
}

}  // namespace pkv
