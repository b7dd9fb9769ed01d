// svq_common.hip -- device entry points of svq.h that are not tied to one
// weight format: the error message, the head's workspace size, greedy
// acceptance of a verified block from ids already computed, and the
// streaming-read probe that measures the HBM read ceiling.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "launch.h"
#include "svq.h"
#include "svq_internal.h"

namespace svq {
char* error_buffer() {
  static thread_local char buf[512];
  return buf;
}
}  // namespace svq

extern "C" const char* svq_last_error(void) { return svq::error_buffer(); }

namespace {

__global__ void __launch_bounds__(64) k_verify_greedy(const int32_t* __restrict__ target,
                                                      const int32_t* __restrict__ draft, int M,
                                                      int32_t* __restrict__ accept) {
  if (threadIdx.x == 0) accept[0] = greedy_accept_len(target, draft, M);
}

// Streaming-read ceiling: every thread keeps U non-temporal 16-byte loads in
// flight over a grid-stride walk of the buffer.  The last partial round
// issues its loads together as well: past the end they read the last element
// again and are dropped, so no load sits behind a branch of its own (a
// guarded load per branch would wait for each load before the next).  One
// checksum per workgroup keeps the loads live.
__global__ void __launch_bounds__(256) k_stream_read(const uint4* __restrict__ src, size_t n16,
                                                     uint32_t* __restrict__ sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    v4u_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (i < n16) {
    v4u_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + u * stride;
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(src + (j < n16 ? j : n16 - 1)));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u * stride < n16) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" {

size_t svq_lmhead_workspace_bytes(int32_t M) {
  if (M < 1 || M > SVQ_MAX_M) return 0;
  return (size_t)kWsBytes;
}

int verify_greedy(const int32_t* target_ids, const int32_t* draft_ids, int32_t M, int32_t* accept_len, void* stream) {
  svq::clear_error();
  if (!target_ids || !accept_len || (M > 1 && !draft_ids))
    return svq::fail(SVQ_ERR_NULL, "verify_greedy: NULL pointer");
  if (M < 1 || M > SVQ_MAX_M) return svq::fail(SVQ_ERR_SHAPE, "verify_greedy: M=%d must be in 1..16", M);
  if (misaligned(target_ids, 4) || misaligned(accept_len, 4) || (draft_ids && misaligned(draft_ids, 4)))
    return svq::fail(SVQ_ERR_ALIGN, "verify_greedy: pointers must be 4-byte aligned");
  hipLaunchKernelGGL(k_verify_greedy, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), target_ids,
                     draft_ids, M, accept_len);
  return launched("verify_greedy");
}

int svq_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t wgs_per_cu, void* stream) {
  svq::clear_error();
  if (!src || !sink) return svq::fail(SVQ_ERR_NULL, "svq_stream_read: NULL pointer");
  if (bytes == 0 || bytes % 16 || bytes >= ((size_t)1 << 31))
    return svq::fail(SVQ_ERR_SHAPE, "svq_stream_read: bytes must be a positive multiple of 16 below 2 GiB");
  if (wgs_per_cu < 0 || wgs_per_cu > 8)
    return svq::fail(SVQ_ERR_SHAPE, "svq_stream_read: wgs_per_cu must be in 0..8 (got %d)", wgs_per_cu);
  if (misaligned(src, 16) || misaligned(sink, 4)) return svq::fail(SVQ_ERR_ALIGN, "svq_stream_read: misaligned pointer");
  int cus = 0;
  if (int rc = device_cus(&cus)) return rc;
  // Eight loads per thread in flight; wgs_per_cu workgroups per CU (0: one,
  // which measured best for large buffers); fewer when the buffer is smaller
  // than one full round.
  const size_t per_wg = (size_t)256 * 16 * 8;
  size_t grid = (bytes + per_wg - 1) / per_wg;
  const size_t cap = (size_t)cus * (wgs_per_cu == 0 ? 1 : wgs_per_cu);
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const uint4*>(src), bytes / 16, sink);
  return launched("svq_stream_read");
}

}  // extern "C"
