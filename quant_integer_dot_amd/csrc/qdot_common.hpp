// qdot_common.hpp -- device-side constants and helpers shared by the HIP
// kernels of libqdot (gfx950 only).  Nothing here is shared with the CPU
// oracle.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace qdot {

// Block geometry (xLLM v0.7 log section 1 and the V100TPS log of 2026-08-12:
// superblocks of 256 weights; Q8_1 activation blocks of 32).
constexpr int QK = 256;          // weights per superblock
constexpr int Q8_BLOCK = 32;     // activations per Q8_1 block
constexpr int Q8_BYTES = 36;     // fp16 d, fp16 s, int8 q[32]
constexpr int QUARTER = 64;      // weights handled by one lane per superblock

enum Type : int { Q4_K = 1, Q6_K = 2, IQ4_XS = 3, Q4_0 = 4, Q8_0 = 5 };

template <int T> struct Geom;
template <> struct Geom<Q4_K>   { static constexpr int BYTES = 144; static constexpr int SUB = 32; };
template <> struct Geom<Q6_K>   { static constexpr int BYTES = 210; static constexpr int SUB = 16; };
template <> struct Geom<IQ4_XS> { static constexpr int BYTES = 136; static constexpr int SUB = 32; };
// Q4_0 / Q8_0: eight consecutive 32-weight blocks stand in for a superblock.
template <> struct Geom<Q4_0>   { static constexpr int BYTES = 8 * 18; static constexpr int SUB = 32; };
template <> struct Geom<Q8_0>   { static constexpr int BYTES = 8 * 34; static constexpr int SUB = 32; };
static_assert(Geom<Q4_K>::BYTES == 4 + 12 + QK / 2, "Q4_K superblock size");
static_assert(Geom<Q6_K>::BYTES == QK / 2 + QK / 4 + QK / 16 + 2, "Q6_K superblock size");
static_assert(Geom<IQ4_XS>::BYTES == 2 + 2 + 4 + QK / 2, "IQ4_XS superblock size");
static_assert(QK % QUARTER == 0 && QUARTER == 2 * Q8_BLOCK, "a lane quarter is two Q8_1 blocks");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-byte global load from any byte address (gfx950 runs HSA in unaligned
// access mode, so this is one global_load_dwordx4).
__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}
__device__ __forceinline__ u32x2 ld8(const uint8_t* p) {
  u32x2 v;
  __builtin_memcpy(&v, p, 8);
  return v;
}
__device__ __forceinline__ uint32_t ld4(const uint8_t* p) {
  uint32_t v;
  __builtin_memcpy(&v, p, 4);
  return v;
}

// binary16 bits -> float (exact, subnormals included).
__device__ __forceinline__ float h2f(uint32_t bits16) {
  return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

// binary16 bits of S = D * sumq for a Q8_1 block.  The product is exact in
// fp32 (11 + 12 significant bits), so S takes one rounding.  A zero product
// keeps its IEEE sign (D = +0 with a negative sum gives -0): the compiler
// would otherwise fold the multiply and the conversion into a mixed-precision
// FMA with a +0 addend, which turns -0 into +0.
__device__ __forceinline__ uint32_t q8_1_s_bits(__half dh, int sumq) {
  const float p = __half2float(dh) * (float)sumq;
  if (p == 0.0f) return (__float_as_uint(p) >> 16) & 0x8000u;
  return __half_as_ushort(__float2half_rn(p));
}

// One Q8_1 block quantized by an aligned group of 8 lanes, 4 values a lane
// (lane part p = lane % 8 holds elements 4p .. 4p+3): amax over the group,
// d32 = amax / 127 (correctly rounded fp32 division; this code must never be
// built with fast-math), q = roundf(v / d32) (fp32 division, ties away from
// zero) clamped to [-127, 127], all zero when amax == 0; d and s stored as
// binary16, s = d * sum q.  Returns this lane's four codes packed little
// endian, the sum of its own four codes, and (in every lane of the group)
// the block's code sum and its d | s << 16 bits.  Every lane of the wave must
// call it (the group reductions are cross-lane shuffles).  The standalone
// quantizer and the decode kernel's in-kernel quantization both use it, so
// their bytes are the same by construction.
__device__ __forceinline__ void q8_1_block8(const float (&v)[4], uint32_t& packed, int& part_sum,
                                            int& sumq, uint32_t& ds) {
  float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  amax = fmaxf(amax, __shfl_xor(amax, 4));
  packed = 0;
  part_sum = 0;
  float d32 = 0.0f;
  if (amax != 0.0f) {
    d32 = amax / 127.0f;  // IEEE-correct fp32 division
    // q = roundf(v / d32) with the correctly rounded quotient, found without
    // a division where that provably gives the same integer: with r the
    // hardware reciprocal of d32 (within 1 ulp) and t = v * r rounded, t is
    // within |v/d32| * 1.5 * 2^-23 <= 2.3e-5 of v/d32 (|v/d32| <= 127.00001),
    // and the rounded quotient within 3.9e-6 of it.  If t is more than 2^-14
    // from every half-integer, all three lie strictly between the same two
    // half-integers, so they round to the same integer, the nearest to t.
    // Otherwise (or for a reciprocal out of range: a NaN or infinite t fails
    // the test) the whole wave takes the correctly rounded division.
    const float rcp = __builtin_amdgcn_rcpf(d32);
    float n[4];
    bool fast = d32 >= 0x1p-100f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t = v[i] * rcp;
      n[i] = __builtin_rintf(t);
      fast = fast && fabsf(t - n[i]) < 0.5f - 0x1p-14f;
    }
    if (__all(fast)) {  // every active lane of the wave can take the fast path
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qi = (int)fminf(fmaxf(n[i], -127.0f), 127.0f);
        part_sum += qi;
        packed |= ((uint32_t)qi & 0xFFu) << (8 * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float r = roundf(v[i] / d32);  // ties away from zero
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        const int qi = (int)r;
        part_sum += qi;
        packed |= ((uint32_t)qi & 0xFFu) << (8 * i);
      }
    }
  }
  sumq = part_sum;
  sumq += __shfl_xor(sumq, 1);
  sumq += __shfl_xor(sumq, 2);
  sumq += __shfl_xor(sumq, 4);
  const __half dh = __float2half_rn(d32);
  ds = (uint32_t)__half_as_ushort(dh) | (q8_1_s_bits(dh, sumq) << 16);
}

// Integer dot of four int8 pairs, accumulated (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
  return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// Bytes 2..5 of the 8-byte pair {hi:lo} (v_alignbyte_b32): the dword that
// starts 2 bytes into lo, for 2-byte-aligned block fields.
__device__ __forceinline__ uint32_t shr16(uint32_t hi, uint32_t lo) {
  return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// Byte permute: byte k of the result is byte sel[k] of {hi:lo} (v_perm_b32).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace qdot
