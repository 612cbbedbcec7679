// Opt-in per-phase timestamps of the decode main loops, for measuring where a
// loop step's time goes. Built only with -DPKV_STAMPS=1 (paged_kv_fp8_amd/
// stamps.py builds such a library beside the normal one and prints the
// phases); in a normal build every macro below is empty.
//
// Lane 0 of each wave (at most kStampWaves) of workgroups 0 .. kStampWgs - 1
// (blockIdx.y = blockIdx.z = 0) reads s_memtime at up to kStampPoints points
// of each of the first kStampSteps steps of its first work item and stores
// them (vector stores) to a per-source device array, which pkv_debug_stamps
// copies out. A scheduling barrier on each side of a stamp keeps the phases
// apart, so a stamped build runs somewhat slower than the normal one, and
// the compiler cannot overlap one phase with the next as it otherwise may.
#pragma once

#include <hip/hip_runtime.h>

namespace pkv {

constexpr int kStampWgs = 16, kStampWaves = 8, kStampSteps = 48, kStampPoints = 8;
constexpr int kStampWords = kStampWgs * kStampWaves * kStampSteps * kStampPoints;

}  // namespace pkv

#if PKV_STAMPS
#define PKV_STAMP_STORAGE static __device__ unsigned long long g_stamps[kStampWords];
#define PKV_STAMP_VARS unsigned long long pkv_ts[kStampPoints] = {};
#define PKV_STAMP(k)                                 \
  do {                                               \
    __builtin_amdgcn_sched_barrier(0);               \
    pkv_ts[k] = __builtin_amdgcn_s_memtime();        \
    __builtin_amdgcn_sched_barrier(0);               \
  } while (0)
// store the step's stamps (first work item of the workgroup only)
#define PKV_STAMP_SAVE(step, first_item)                                                                         \
  do {                                                                                                           \
    const int pkv_w = (int)(threadIdx.x >> 6);                                                                   \
    if ((first_item) && blockIdx.x < kStampWgs && blockIdx.y == 0 && blockIdx.z == 0 && pkv_w < kStampWaves &&   \
        (step) >= 0 && (step) < kStampSteps && (threadIdx.x & 63) == 0)                                          \
      for (int pkv_k = 0; pkv_k < kStampPoints; ++pkv_k)                                                         \
        g_stamps[((blockIdx.x * kStampWaves + pkv_w) * kStampSteps + (step)) * kStampPoints + pkv_k] = pkv_ts[pkv_k]; \
  } while (0)
#define PKV_STAMP_COPY(dst) hipMemcpyFromSymbol((dst), HIP_SYMBOL(g_stamps), sizeof(g_stamps))
#else
#define PKV_STAMP_STORAGE
#define PKV_STAMP_VARS
#define PKV_STAMP(k) \
  do {               \
  } while (0)
#define PKV_STAMP_SAVE(step, first_item) \
  do {                                   \
  } while (0)
#define PKV_STAMP_COPY(dst) hipErrorNotSupported
#endif
