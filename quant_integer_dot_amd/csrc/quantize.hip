// quantize.hip -- fp32 activations -> Q8_1 blocks (row a1 of the hot path).
//
// The pages launch quantize_q8_1 once ahead of the integer-dot matmul and
// share its output across every row of the batch (V100TPS log, 2026-08-12,
// ggml_mul_mat_a8; xLLM v0.7 log, section C, the shared d_xn_q8 buffer).  The
// rounding is not stated there; this kernel implements the reading documented
// in qdot.h: d32 = amax/127 and q = roundf(x/d32) with correctly rounded fp32
// division (this file must never be built with fast-math), d and s stored as
// binary16 round-to-nearest-even, s = d*sum(q).
//
// Mapping: 8 lanes per 32-element block, 4 floats per lane (one 16-byte
// load); amax and sum(q) are reduced over the 8 lanes with xor shuffles
// (q8_1_block8, shared with the decode kernel's in-kernel quantization).  The
// kernel is HBM-bound (4 B read, 1.125 B written per element).
#include "qdot_common.hpp"

namespace qdot {

__global__ __launch_bounds__(256) void quantize_q8_1_kernel(
    const float* __restrict__ x, int64_t nblocks, uint8_t* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = gid >> 3;      // Q8_1 block index over [M][K/32]
  const int part = (int)(gid & 7);   // which 4 floats of the block
  const bool live = blk < nblocks;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    u32x4 raw = ld16(reinterpret_cast<const uint8_t*>(x + blk * Q8_BLOCK + part * 4));
    v[0] = __uint_as_float(raw.x);
    v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z);
    v[3] = __uint_as_float(raw.w);
  }
  uint32_t packed, ds;
  int part_sum, sumq;
  q8_1_block8(v, packed, part_sum, sumq, ds);
  if (!live) return;

  uint8_t* ob = out + blk * Q8_BYTES;
  *reinterpret_cast<uint32_t*>(ob + 4 + 4 * part) = packed;
  if (part == 0) *reinterpret_cast<uint32_t*>(ob) = ds;
}

int launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* xq, hipStream_t s) {
  const int64_t nblocks = M * (K / Q8_BLOCK);
  const int64_t threads = nblocks * 8;
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(quantize_q8_1_kernel, dim3((unsigned)grid), dim3(256), 0, s, x, nblocks,
                     static_cast<uint8_t*>(xq));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace qdot
