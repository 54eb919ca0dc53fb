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
