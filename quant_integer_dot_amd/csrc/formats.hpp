// formats.hpp -- device helpers for the weight block formats, shared by every
// kernel of libqdot (decode, mid-batch, prefill): the one definition of each
// field unpacking, so a layout reading lives in one place.  Nothing here is
// shared with the CPU oracle.
//
// Layout readings (the pages name the formats but print no layouts; these are
// the plain GGUF readings):
//   Q4_K   bytes 0-1 d, 2-3 dmin, 4-15 scales[12] (six-bit scale and min of
//          eight 32-element sub-blocks), 16-143 codes;
//   Q6_K   0-127 low four bits, 128-191 high two bits, 192-207 int8
//          sub-scales of sixteen 16-element sub-blocks, 208-209 d;
//   IQ4_XS 0-1 d, 2-3 scales_h, 4-7 scales_l, 8-135 four-bit indices into
//          the IQ4_NL codebook (V100TPS log, 2026-08-12 entries: scale
//          d*(ls-32), codebook values instead of q-8);
//   Q4_0   per 32 weights fp16 d and 16 bytes of nibbles, value d*(q-8).
#pragma once

#include "qdot_common.hpp"

namespace qdot {

// IQ4_NL codebook as four little-endian dwords (entries 0-3, 4-7, 8-11,
// 12-15).  Placeholder values (the pages name kvalues_iq4nl without printing
// it): round_half_away(-127 + 240*(i/15)^1.4).
//   -127 -122 -113 -102 | -89 -75 -60 -44 | -27 -10 9 28 | 49 69 91 113
constexpr uint32_t CB0 = 0x9A8F8681u;  // 0x81=-127 0x86=-122 0x8F=-113 0x9A=-102
constexpr uint32_t CB1 = 0xD4C4B5A7u;  // 0xA7=-89 0xB5=-75 0xC4=-60 0xD4=-44
constexpr uint32_t CB2 = 0x1C09F6E5u;  // 0xE5=-27 0xF6=-10 0x09=9 0x1C=28
constexpr uint32_t CB3 = 0x715B4531u;  // 0x31=49 0x45=69 0x5B=91 0x71=113

// Four 4-bit indices (the low nibble of each byte; the high nibbles are
// ignored) -> four int8 codebook values: two v_perm lookups on entries 0-7
// and 8-15, then a v_perm that picks, per byte, the first or the second
// result by bit 3 of the index.
__device__ __forceinline__ uint32_t iq4nl_lookup(uint32_t idx) {
  const uint32_t sel = idx & 0x07070707u;
  const uint32_t lo = perm(CB1, CB0, sel);
  const uint32_t hi = perm(CB3, CB2, sel);
  const uint32_t pick = ((idx >> 1) & 0x04040404u) | 0x03020100u;
  return perm(hi, lo, pick);
}

// Q4_K: six-bit scale and min of sub-block j from the header dwords h (h.x =
// d | dmin << 16, h.y .. h.w = scales[0..11]).  j < 4: low six bits of bytes
// j and j+4; j >= 4: the nibbles of byte j+4 below the top two bits of bytes
// j-4 (scale) and j (min).
__device__ __forceinline__ void q4k_scale_min(const u32x4& h, int j, uint32_t& sc, uint32_t& m) {
  const int sh = 8 * (j & 3);
  const uint32_t Ys = h.y >> sh, Zs = h.z >> sh, Ws = h.w >> sh;
  const bool lo = j < 4;
  sc = lo ? (Ys & 63u) : ((Ws & 15u) | ((Ys >> 2) & 0x30u));
  m = lo ? (Zs & 63u) : (((Ws >> 4) & 15u) | ((Zs >> 2) & 0x30u));
}

// Q4_K: d*sc and -dmin*m of sub-block j as fp64; both products are exact in
// fp32 (11 + 6 significant bits).
__device__ __forceinline__ void q4k_scales(const u32x4& h, int j, double& wsc, double& wmn) {
  uint32_t sc, m;
  q4k_scale_min(h, j, sc, m);
  wsc = (double)(h2f(h.x) * (float)sc);
  wmn = -(double)(h2f(h.x >> 16) * (float)m);
}

// IQ4_XS: six-bit scale ls of sub-block j (hx = d | scales_h << 16, hy =
// scales_l): the nibble j of scales_l below bits 2j, 2j+1 of scales_h.
__device__ __forceinline__ int iq4xs_ls(uint32_t hx, uint32_t hy, int j) {
  return (int)(((hy >> (4 * j)) & 15u) | ((((hx >> 16) >> (2 * j)) & 3u) << 4));
}

// IQ4_XS: d*(ls-32) of sub-block j as fp64, exact in fp32.
__device__ __forceinline__ double iq4xs_scale(uint32_t hx, uint32_t hy, int j) {
  return (double)(h2f(hx) * (float)(iq4xs_ls(hx, hy, j) - 32));
}

// Q6_K: four six-bit codes (0..63, one per byte) of group g = gp + 2 * HI
// (gp = 0, 1) of a 128-element half: the low four bits are the low (HI = 0)
// or high (HI = 1) nibbles of the ql dword, the high two bits are bits 2g,
// 2g+1 of the qh dword.
template <int HI>
__device__ __forceinline__ uint32_t q6k_code(uint32_t ql, uint32_t qh, int gp) {
  if constexpr (HI) return ((ql >> 4) & 0x0F0F0F0Fu) | ((qh >> (2 * gp)) & 0x30303030u);
  else return (ql & 0x0F0F0F0Fu) | ((qh << (4 - 2 * gp)) & 0x30303030u);
}

// Q6_K: four six-bit codes (0..63, one per byte) -> int8 code - 32.  With
// bit 7 of each byte set first, the subtraction cannot borrow across bytes
// (128 + c - 32 >= 96), and flipping bit 7 back leaves c - 32 modulo 256.
__device__ __forceinline__ uint32_t q6k_signed(uint32_t u) {
  return ((u | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
}

// Q6_K: the exact integer s0*I0 + s1*I1 of two 16-element sub-blocks (int8
// sub-scales s, sub-block sums I of 16 codes |c - 32| <= 32 against |q| <=
// 127, so |I| <= 65024 and |s*I| < 2^23) on the full-rate 24-bit multipliers
// (v_mul_i32_i24, v_mad_i32_i24).  Written as a plain int expression it
// compiles to v_mul_lo_u32 and v_mad_u64_u32, four times slower.
__device__ __forceinline__ int q6k_pair(int s0, int I0, int s1, int I1) {
  return __mul24(s0, I0) + __mul24(s1, I1);
}

// Q4_0: four nibble codes (0..15, one per byte) -> int8 code - 8, without
// borrows between bytes.
__device__ __forceinline__ uint32_t q40_signed(uint32_t v) {
  return ((v | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}

}  // namespace qdot
