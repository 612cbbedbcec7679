// Latent-record (MLA-like) decode: not built yet; the entry points reject
// PKV_KV_MLA with PKV_ERR_UNSUPPORTED before reaching these launchers.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {

int mla_rows_per_tile(const pkv_decode_args&) { return 16; }

hipError_t mla_occupancy(const pkv_decode_args&, int* wg_per_cu) {
  *wg_per_cu = 1;
  return hipSuccess;
}

hipError_t mla_launch(const pkv_decode_args&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pkv
