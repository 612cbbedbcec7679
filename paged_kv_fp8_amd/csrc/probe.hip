// Streaming-read probe: the HBM read rate this part reaches with plain
// coalesced 16-byte vector loads and no other work, the ceiling against which
// the decode kernels' achieved rate is read as a fraction of what is
// achievable (the t5_decode page's `run` harness reports GB/s = bytes /
// time; this probe gives the same figure for a kernel that only reads).
//
// Grid-stride over chunks of 256 * UNROLL 16-byte words: chunk c is read by
// workgroup c mod grid, each lane issuing UNROLL independent loads (lane l,
// load u reads word c * 256 * UNROLL + u * 256 + l, so every load instruction
// of the workgroup covers 4 KiB of contiguous bytes) before it folds them into
// an XOR. The XOR keeps the loads live; its value is stored only if it equals
// a fixed pattern, so the kernel writes (almost) nothing.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kProbeThreads = 256;

template <int UNROLL>
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ src, int64_t chunks,
                                                                     uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const uint4* base = src + c * (kProbeThreads * UNROLL) + lane;
    uint4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = base[u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t probe_launch(const void* src, size_t bytes, int workgroups, int unroll, uint32_t* sink,
                        hipStream_t stream) {
  const int64_t chunks = (int64_t)(bytes / (16u * kProbeThreads * unroll));
  const dim3 grid(workgroups), block(kProbeThreads);
  const uint4* s = static_cast<const uint4*>(src);
  switch (unroll) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, grid, block, 0, stream, s, chunks, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, grid, block, 0, stream, s, chunks, sink); break;
    default: hipLaunchKernelGGL(stream_read_kernel<16>, grid, block, 0, stream, s, chunks, sink); break;
  }
  return hipGetLastError();
}

}  // namespace pkv
