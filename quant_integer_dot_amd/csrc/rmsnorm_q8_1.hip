// rmsnorm_q8_1.hip -- RMSNorm fused with the Q8_1 quantizer: the producer of
// the activations the Q/K/V and gate/up matmuls read, in one launch instead
// of a norm launch followed by a quantize launch (the xLLM engine keeps one
// quantized normalized-input buffer per step, d_xn_q8, section C.1).
//
// Numerics as the Kestrel_VLLM #18 page gives them (section 3.6, its
// CPU-order RMSNorm kernel and the first row of its table): fp32 throughout;
// each group of 8 consecutive squares s_0..s_7 summed as (lo0 + lo1) +
// (lo2 + lo3) with lo_k = s_k + s_(k+4); the group sums added left to right
// into one accumulator (the page's fix for a GPU tree reduction that broke
// bitwise agreement with the CPU); r = 1.0f / sqrtf(ss / K + eps) with
// correctly rounded division and square root (never an rsqrt
// approximation); out = (x * r) * w.  FMA contraction is off in this file, so
// every operation rounds once, as written.  The normalized values then go
// through the quantizer's own reading (amax/127, roundf(x/d32), fp16 D and S).
//
// Mapping: one workgroup per row, thread b owns Q8_1 block b (32 elements,
// four groups of 8; K <= 32768).  The group sums are formed in parallel and
// staged in LDS; one thread then adds all K/8 of them in order (the only
// serial part: K/8 dependent fp32 adds, its LDS reads issued well ahead),
// and every thread normalizes and quantizes its own block.
#include "qdot_common.hpp"

#pragma clang fp contract(off)

namespace qdot {

constexpr int RN_MAX_THREADS = 1024;
constexpr int RN_AHEAD = 12;  // LDS reads in flight ahead of the serial sum (lgkmcnt counts to 15)

__global__ __launch_bounds__(RN_MAX_THREADS) void rmsnorm_q8_1_kernel(
    const float* __restrict__ x, const float* __restrict__ w, float eps, int K,
    uint8_t* __restrict__ out) {
  __shared__ float4 group_sums[RN_MAX_THREADS];  // block b's four group sums
  __shared__ float r_shared;
  const int m = blockIdx.x;
  const int b = threadIdx.x;
  const int nb = K / Q8_BLOCK;
  const bool live = b < nb;

  float v[Q8_BLOCK];
  u32x4 wr[Q8_BLOCK / 4];  // this block's weights, loaded with x (one memory round trip)
  if (live) {
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(x + (size_t)m * K + (size_t)b * Q8_BLOCK);
    const uint8_t* wb = reinterpret_cast<const uint8_t*>(w + (size_t)b * Q8_BLOCK);
#pragma unroll
    for (int i = 0; i < Q8_BLOCK / 4; ++i) {
      const u32x4 raw = ld16(xb + 16 * i);
      wr[i] = ld16(wb + 16 * i);
      v[4 * i] = __uint_as_float(raw.x);
      v[4 * i + 1] = __uint_as_float(raw.y);
      v[4 * i + 2] = __uint_as_float(raw.z);
      v[4 * i + 3] = __uint_as_float(raw.w);
    }
    float t[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float s0 = v[8 * g + k] * v[8 * g + k];
        const float s1 = v[8 * g + k + 4] * v[8 * g + k + 4];
        lo[k] = s0 + s1;
      }
      const float s01 = lo[0] + lo[1];
      const float s23 = lo[2] + lo[3];
      t[g] = s01 + s23;
    }
    group_sums[b] = make_float4(t[0], t[1], t[2], t[3]);
  }
  __syncthreads();
  if (b == 0) {
    // The groups in order, one accumulator.  The chain of K/8 dependent adds
    // is the kernel's serial part; the LDS reads run RN_AHEAD blocks ahead of
    // it (buf[j] holds block i + j) so that no add waits for a read.
    float ss = 0.0f;
    float4 buf[RN_AHEAD];
#pragma unroll
    for (int j = 0; j < RN_AHEAD; ++j) buf[j] = group_sums[j < nb ? j : nb - 1];
    int i = 0;
    for (; i + RN_AHEAD <= nb; i += RN_AHEAD) {
#pragma unroll
      for (int j = 0; j < RN_AHEAD; ++j) {
        const float4 g = buf[j];
        ss = ss + g.x;
        ss = ss + g.y;
        ss = ss + g.z;
        ss = ss + g.w;
        const int nx = i + j + RN_AHEAD;
        buf[j] = group_sums[nx < nb ? nx : nb - 1];
      }
    }
#pragma unroll
    for (int j = 0; j < RN_AHEAD; ++j) {
      if (j < nb - i) {  // the last nb - i blocks, already in buf
        const float4 g = buf[j];
        ss = ss + g.x;
        ss = ss + g.y;
        ss = ss + g.z;
        ss = ss + g.w;
      }
    }
    const float mean = ss / (float)K;
    r_shared = 1.0f / sqrtf(mean + eps);
  }
  __syncthreads();
  if (!live) return;
  const float r = r_shared;

  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < Q8_BLOCK / 4; ++i) {
    const float wv[4] = {__uint_as_float(wr[i].x), __uint_as_float(wr[i].y), __uint_as_float(wr[i].z),
                         __uint_as_float(wr[i].w)};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = v[4 * i + k] * r;
      v[4 * i + k] = a * wv[k];
      amax = fmaxf(amax, fabsf(v[4 * i + k]));
    }
  }

  uint32_t packed[Q8_BLOCK / 4];
  int sumq = 0;
  float d32 = 0.0f;
#pragma unroll
  for (int i = 0; i < Q8_BLOCK / 4; ++i) packed[i] = 0;
  if (amax != 0.0f) {
    d32 = amax / 127.0f;  // IEEE-correct fp32 division
#pragma unroll
    for (int i = 0; i < Q8_BLOCK; ++i) {
      float q = roundf(v[i] / d32);  // ties away from zero
      q = fminf(fmaxf(q, -127.0f), 127.0f);
      const int qi = (int)q;
      sumq += qi;
      packed[i >> 2] |= ((uint32_t)qi & 0xFFu) << (8 * (i & 3));
    }
  }
  uint8_t* ob = out + ((size_t)m * nb + b) * Q8_BYTES;
  const __half dh = __float2half_rn(d32);
  *reinterpret_cast<uint32_t*>(ob) = (uint32_t)__half_as_ushort(dh) | (q8_1_s_bits(dh, sumq) << 16);
#pragma unroll
  for (int i = 0; i < Q8_BLOCK / 4; ++i) *reinterpret_cast<uint32_t*>(ob + 4 + 4 * i) = packed[i];
}

int launch_rmsnorm_q8_1(const float* x, const float* w, float eps, int64_t M, int64_t K, void* xq,
                        hipStream_t s) {
  const int nb = (int)(K / Q8_BLOCK);
  const int threads = (nb + 63) / 64 * 64;
  if (threads > RN_MAX_THREADS || M > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(rmsnorm_q8_1_kernel, dim3((unsigned)M), dim3(threads), 0, s, x, w, eps, (int)K,
                     static_cast<uint8_t*>(xq));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace qdot
