// stream_ref.hip -- a plain read-only streaming kernel: the memory system's
// reference rate for the HBM-bound decode launches.  It reads a buffer once
// with coalesced 16-byte loads (four per thread, all in flight together) and
// keeps only an XOR fold of what it read, so it moves the same kind of bytes
// as a decode launch with no arithmetic and (almost) no writes.  Not on the
// matmul path; the benchmark times it at the dominant launch's size.
#include "qdot_common.hpp"

namespace qdot {

constexpr int SR_THREADS = 256;
constexpr int SR_PER_THREAD = 4;  // 16-byte loads per thread

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * SR_THREADS * SR_PER_THREAD + threadIdx.x;
  u32x4 v[SR_PER_THREAD];
#pragma unroll
  for (int k = 0; k < SR_PER_THREAD; ++k) {
    const int64_t i = base + (int64_t)k * SR_THREADS;
    v[k] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < SR_PER_THREAD; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  // The fold decides a store that practically never happens, so the loads
  // cannot be dropped; sink holds one dword.
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (int64_t)SR_THREADS * SR_PER_THREAD;
  const int64_t grid = (n16 + per_block - 1) / per_block;
  if (grid < 1 || grid > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(SR_THREADS), 0, s,
                     static_cast<const u32x4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace qdot
