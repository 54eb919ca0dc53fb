// qmv.hip -- decode matmul for M = 1..8 token rows (rows a2-a5 of the hot
// path): y[m][n] = sum_k w[n][k] * xhat[m][k] on the raw Q4_K / Q6_K / IQ4_XS
// superblocks, with v_dot4_i32_i8 integer dots against Q8_1 activations.
//
// What the pages fix, and what this kernel keeps:
//  * integer dots on the raw quantized weights, fp32 out, no fp32 weight copy
//    (xLLM v0.7 log, section 1);
//  * an M-row tile, so each weight byte is read from HBM once for all M rows
//    (xLLM section B2, q4k_dp4a_matmul_q8_v2_kernel<M>; V100TPS 2026-08-12,
//    "batched MMVQ: weights read once, not once per token position");
//  * the weight decode and the IQ4_NL lookup done once per weight, not once per
//    row (V100TPS 2026-08-12: moving the kvalues lookup to load time gave 1.5x);
//  * exact int32 sums inside each sub-block, scales applied afterwards
//    (Kestrel section 5).
// What differs from the pages' V100 design: the M=8 V100 kernel was L1-bound
// (xLLM section B2 ncu table).  Here the activations of a K-chunk are staged
// once per workgroup into LDS (int8 codes plus fp64 scales), each lane keeps
// the activation dwords of its current block in VGPRs and reuses them for R
// weight rows, and the scale drains are exact fp64 terms (every product exact,
// one rounding per accumulate), so y is the fp32 rounding of a value within a
// few fp64 ulps of the exact sum.
//
// Mapping (256 threads = 4 waves of 64):
//  * lane = (slot s = lane/4, quarter q = lane%4).  A quarter is 64 weights of
//    a superblock = two Q8_1 activation blocks, in all three formats;
//  * the workgroup owns rows n0 + s + 16*r (r < R): 16*R rows;
//  * wave w takes superblocks b = w, w+4, ... of the current K-chunk;
//  * the partial sums are reduced over the 4 quarter lanes (xor shuffles), then
//    over the 4 waves through LDS in a fixed order (deterministic, and the same
//    for every M: row m of y does not depend on M).
#include "qdot_common.hpp"

namespace qdot {

constexpr int QMV_THREADS = 256;
constexpr int QMV_WAVES = 4;
constexpr int QMV_SLOTS = 16;  // row slots per wave (64 lanes / 4 quarters)

// One LDS entry per Q8_1 block and row m: the fp64 scale D and a second field
// (Q4_K: fp64 S; Q6_K: 32 * sum of each 16-element half of q; IQ4_XS: unused).
struct __attribute__((aligned(16))) DsEntry {
  double d;
  union {
    double s;
    int xs32[2];
  };
};
static_assert(sizeof(DsEntry) == 16, "DsEntry is 16 bytes");

// --------------------------------------------------------------- formats
template <int T> struct Fmt;

// Q4_K: bytes 0-1 d, 2-3 dmin, 4-15 scales[12], 16-143 qs.  Quarter q holds
// qs[32q .. 32q+31]: low nibbles = sub-block 2q, high nibbles = sub-block 2q+1.
template <> struct Fmt<Q4_K> {
  struct Regs { u32x4 h, a, b; };
  __device__ static Regs load(const uint8_t* sb, int q) {
    Regs r;
    r.h = ld16(sb);
    r.a = ld16(sb + 16 + 32 * q);
    r.b = ld16(sb + 32 + 32 * q);
    return r;
  }
  // Q8_1 blocks (within the superblock) used by quarter q, and which sub-block
  // of the superblock each is.
  __device__ static int blk(int q, int half) { return 2 * q + half; }
};

// Q6_K: bytes 0-127 ql, 128-191 qh, 192-207 int8 scales, 208-209 d.  Quarter
// q = (h = q/2, gp = q%2) holds ql[64h + 32gp ..+32] and qh[32h ..+32]: low
// nibbles = Q8 block 4h+gp, high nibbles = Q8 block 4h+gp+2.
template <> struct Fmt<Q6_K> {
  struct Regs { u32x4 a, b, c, e, sc; uint32_t d; };
  __device__ static Regs load(const uint8_t* sb, int q) {
    const int h = q >> 1, gp = q & 1;
    Regs r;
    r.a = ld16(sb + 64 * h + 32 * gp);
    r.b = ld16(sb + 64 * h + 32 * gp + 16);
    r.c = ld16(sb + 128 + 32 * h);
    r.e = ld16(sb + 128 + 32 * h + 16);
    r.sc = ld16(sb + 192);
    unsigned short dh;
    __builtin_memcpy(&dh, sb + 208, 2);
    r.d = dh;
    return r;
  }
  __device__ static int blk(int q, int half) { return 4 * (q >> 1) + (q & 1) + 2 * half; }
};

// IQ4_XS: bytes 0-1 d, 2-3 scales_h, 4-7 scales_l, 8-135 qs.  Quarter q holds
// qs[32q .. 32q+31] = sub-blocks 2q (bytes 0-15) and 2q+1 (bytes 16-31); in
// each, low nibbles are elements 0-15 and high nibbles elements 16-31.
template <> struct Fmt<IQ4_XS> {
  struct Regs { u32x2 h; u32x4 a, b; };
  __device__ static Regs load(const uint8_t* sb, int q) {
    Regs r;
    r.h = ld8(sb);
    r.a = ld16(sb + 8 + 32 * q);
    r.b = ld16(sb + 24 + 32 * q);
    return r;
  }
  __device__ static int blk(int q, int half) { return 2 * q + half; }
};

// IQ4_NL-style codebook as four little-endian dwords (entries 0-3, 4-7, 8-11,
// 12-15).  Placeholder values (the pages name kvalues_iq4nl without printing
// it): round_half_away(-127 + 240*(i/15)^1.4).
//   -127 -122 -113 -102 | -89 -75 -60 -44 | -27 -10 9 28 | 49 69 91 113
constexpr uint32_t CB0 = 0x9A8F8681u;  // 0x81=-127 0x86=-122 0x8F=-113 0x9A=-102
constexpr uint32_t CB1 = 0xD4C4B5A7u;  // 0xA7=-89 0xB5=-75 0xC4=-60 0xD4=-44
constexpr uint32_t CB2 = 0x1C09F6E5u;  // 0xE5=-27 0xF6=-10 0x09=9 0x1C=28
constexpr uint32_t CB3 = 0x715B4531u;  // 0x31=49 0x45=69 0x5B=91 0x71=113

// Four 4-bit indices (one per byte, values 0..15) -> four int8 codebook
// values: two v_perm lookups on entries 0-7 and 8-15, then a v_perm that
// picks, per byte, the first or the second result by bit 3 of the index.
__device__ __forceinline__ uint32_t cb_lookup(uint32_t idx, uint32_t t0, uint32_t t1,
                                              uint32_t t2, uint32_t t3) {
  const uint32_t sel = idx & 0x07070707u;
  const uint32_t lo = perm(t1, t0, sel);
  const uint32_t hi = perm(t3, t2, sel);
  const uint32_t pick = ((idx >> 1) & 0x04040404u) | 0x03020100u;
  return perm(hi, lo, pick);
}

// ---------------------------------------------------------------- kernel
template <int T, int M, int R, bool DUMP>
__global__ __launch_bounds__(QMV_THREADS) void qmv_dot4_kernel(
    const uint8_t* __restrict__ W, int N, int K, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ isums, int kc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int SUB = Geom<T>::SUB;
  const int nsb = K / QK;                  // superblocks per row
  const size_t row_bytes = (size_t)nsb * BYTES;
  const int nq8 = K / Q8_BLOCK;            // Q8_1 blocks per activation row

  uint8_t* lds_x = smem;                                   // int8 [M][kc]
  DsEntry* lds_ds = reinterpret_cast<DsEntry*>(smem + (size_t)M * kc);  // [M][kc/32]
  double* lds_red = reinterpret_cast<double*>(smem + (size_t)M * kc + (size_t)M * (kc / 32) * sizeof(DsEntry));

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane >> 2;
  const int q = lane & 3;
  const int n0 = blockIdx.x * (QMV_SLOTS * R);

  // Rows of this lane; rows past N re-read row N-1 and are never stored.
  const uint8_t* wrow[R];
  int nrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    nrow[r] = n0 + slot + QMV_SLOTS * r;
    const int nc = nrow[r] < N ? nrow[r] : N - 1;
    wrow[r] = W + (size_t)nc * row_bytes;
  }

  double acc[R][M];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.0;

  for (int c0 = 0; c0 < K; c0 += kc) {
    const int kcc = (K - c0) < kc ? (K - c0) : kc;
    const int nblk = kcc / Q8_BLOCK;
    __syncthreads();
    // ---- stage the chunk's activations: int8 codes and fp64 scales
    for (int it = tid; it < M * nblk; it += QMV_THREADS) {
      const int m = it / nblk, kb = it - m * nblk;
      const uint8_t* src = xq + ((size_t)m * nq8 + c0 / Q8_BLOCK + kb) * Q8_BYTES;
      const uint32_t ds = ld4(src);
      const u32x4 q0 = ld16(src + 4), q1 = ld16(src + 20);
      *reinterpret_cast<u32x4*>(lds_x + (size_t)m * kc + Q8_BLOCK * kb) = q0;
      *reinterpret_cast<u32x4*>(lds_x + (size_t)m * kc + Q8_BLOCK * kb + 16) = q1;
      DsEntry e;
      e.d = (double)h2f(ds & 0xFFFFu);
      if (T == Q6_K) {
        const uint32_t ones = 0x01010101u;
        const int lo = dot4(q0.w, ones, dot4(q0.z, ones, dot4(q0.y, ones, dot4(q0.x, ones, 0))));
        const int hi = dot4(q1.w, ones, dot4(q1.z, ones, dot4(q1.y, ones, dot4(q1.x, ones, 0))));
        e.xs32[0] = 32 * lo;
        e.xs32[1] = 32 * hi;
      } else {
        e.s = (double)h2f(ds >> 16);
      }
      lds_ds[(size_t)m * (kc / 32) + kb] = e;
    }
    __syncthreads();

    const int nsb_c = kcc / QK;
    const int sb0 = c0 / QK;
    for (int bl = wave; bl < nsb_c; bl += QMV_WAVES) {
      const int b = sb0 + bl;
      typename Fmt<T>::Regs rg[R];
#pragma unroll
      for (int r = 0; r < R; ++r) rg[r] = Fmt<T>::load(wrow[r] + (size_t)b * BYTES, q);

#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = bl * (QK / Q8_BLOCK) + Fmt<T>::blk(q, half);  // chunk-local Q8 block
        uint32_t xa[M][8];
        DsEntry de[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 v0 = *reinterpret_cast<const u32x4*>(lds_x + (size_t)m * kc + Q8_BLOCK * kb);
          const u32x4 v1 = *reinterpret_cast<const u32x4*>(lds_x + (size_t)m * kc + Q8_BLOCK * kb + 16);
          xa[m][0] = v0.x; xa[m][1] = v0.y; xa[m][2] = v0.z; xa[m][3] = v0.w;
          xa[m][4] = v1.x; xa[m][5] = v1.y; xa[m][6] = v1.z; xa[m][7] = v1.w;
          de[m] = lds_ds[(size_t)m * (kc / 32) + kb];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const typename Fmt<T>::Regs& g = rg[r];
          if constexpr (T == Q4_K) {
            // sub-block j = 2q + half: 6-bit scale and min (plain GGUF packing)
            const int p = (2 * q) & 3;
            const uint32_t Ys = g.h.y >> (8 * p), Zs = g.h.z >> (8 * p), Ws = g.h.w >> (8 * p);
            const int sh = 8 * half;
            uint32_t sc, mn;
            if (q < 2) {
              sc = (Ys >> sh) & 63u;
              mn = (Zs >> sh) & 63u;
            } else {
              sc = ((Ws >> sh) & 15u) | ((Ys >> (sh + 2)) & 0x30u);
              mn = ((Ws >> (sh + 4)) & 15u) | ((Zs >> (sh + 2)) & 0x30u);
            }
            const double wsc = (double)(h2f(g.h.x) * (float)sc);          // d*sc, exact
            const double wmn = -(double)(h2f(g.h.x >> 16) * (float)mn);   // -dmin*m, exact
            const uint32_t pk[8] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w};
            uint32_t cw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) cw[i] = (half ? (pk[i] >> 4) : pk[i]) & 0x0F0F0F0Fu;
#pragma unroll
            for (int m = 0; m < M; ++m) {
              int I = 0;
#pragma unroll
              for (int i = 0; i < 8; ++i) I = dot4(cw[i], xa[m][i], I);
              acc[r][m] = fma(wsc * de[m].d, (double)I, acc[r][m]);
              acc[r][m] = fma(wmn, de[m].s, acc[r][m]);
              if (DUMP && nrow[r] < N)
                isums[((size_t)m * N + nrow[r]) * (K / SUB) + (size_t)b * (QK / SUB) + 2 * q + half] = I;
            }
          } else if constexpr (T == IQ4_XS) {
            const int j = 2 * q + half;
            const uint32_t sl = (g.h.y >> (4 * j)) & 15u;
            const uint32_t shb = ((g.h.x >> 16) >> (2 * j)) & 3u;
            const int ls = (int)(sl | (shb << 4));
            const double wsc = (double)(h2f(g.h.x) * (float)(ls - 32));  // d*(ls-32), exact
            const u32x4 pq = half ? g.b : g.a;
            const uint32_t pk[4] = {pq.x, pq.y, pq.z, pq.w};
            uint32_t cw[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              cw[i] = cb_lookup(pk[i], CB0, CB1, CB2, CB3);              // elements 4i..4i+3
              cw[i + 4] = cb_lookup(pk[i] >> 4, CB0, CB1, CB2, CB3);     // elements 16+4i..
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
              int I = 0;
#pragma unroll
              for (int i = 0; i < 8; ++i) I = dot4(cw[i], xa[m][i], I);
              acc[r][m] = fma(wsc * de[m].d, (double)I, acc[r][m]);
              if (DUMP && nrow[r] < N)
                isums[((size_t)m * N + nrow[r]) * (K / SUB) + (size_t)b * (QK / SUB) + j] = I;
            }
          } else {  // Q6_K
            const int h = q >> 1, gp = q & 1;
            // codes for Q8 block (half 0: g = gp from low nibbles; half 1:
            // g = gp+2 from high nibbles); values 0..63, the -32 offset is
            // applied through the activation sums.
            const uint32_t pl[8] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w};
            const uint32_t ph[8] = {g.c.x, g.c.y, g.c.z, g.c.w, g.e.x, g.e.y, g.e.z, g.e.w};
            uint32_t cw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              if (half == 0)
                cw[i] = (pl[i] & 0x0F0F0F0Fu) | ((ph[i] << (4 - 2 * gp)) & 0x30303030u);
              else
                cw[i] = ((pl[i] >> 4) & 0x0F0F0F0Fu) | ((ph[i] >> (2 * gp)) & 0x30303030u);
            }
            // int8 sub-scales of sub-blocks t0 = 8h + 2gp + 4*half and t0 + 1
            const uint32_t scw = h ? (half ? g.sc.w : g.sc.z) : (half ? g.sc.y : g.sc.x);
            const int s0 = (int)(int8_t)(scw >> (16 * gp));
            const int s1 = (int)(int8_t)(scw >> (16 * gp + 8));
            const float d = h2f(g.d);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              int I0 = 0, I1 = 0;
#pragma unroll
              for (int i = 0; i < 4; ++i) I0 = dot4(cw[i], xa[m][i], I0);
#pragma unroll
              for (int i = 4; i < 8; ++i) I1 = dot4(cw[i], xa[m][i], I1);
              I0 -= de[m].xs32[0];
              I1 -= de[m].xs32[1];
              const int P = s0 * I0 + s1 * I1;
              acc[r][m] = fma((double)d * de[m].d, (double)P, acc[r][m]);
              if (DUMP && nrow[r] < N) {
                const size_t base = ((size_t)m * N + nrow[r]) * (K / SUB) + (size_t)b * (QK / SUB) +
                                    8 * h + 2 * gp + 4 * half;
                isums[base] = I0;
                isums[base + 1] = I1;
              }
            }
          }
        }
      }
    }
  }

  // ---- reduce over the 4 quarter lanes, then over the 4 waves
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      double v = acc[r][m];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      acc[r][m] = v;
    }
  __syncthreads();
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        lds_red[((wave * QMV_SLOTS + slot) * R + r) * M + m] = acc[r][m];
  }
  __syncthreads();
  for (int o = tid; o < QMV_SLOTS * R * M; o += QMV_THREADS) {
    const int m = o % M;
    const int r = (o / M) % R;
    const int s = o / (M * R);
    const int n = n0 + s + QMV_SLOTS * r;
    double v = lds_red[((0 * QMV_SLOTS + s) * R + r) * M + m];
#pragma unroll
    for (int w = 1; w < QMV_WAVES; ++w) v += lds_red[((w * QMV_SLOTS + s) * R + r) * M + m];
    if (n < N) y[(size_t)m * N + n] = (float)v;
  }
}

// ------------------------------------------------------------- launcher
template <int M> struct QmvCfg { static constexpr int R = 2; };

// LDS budget per workgroup for the activation chunk.
constexpr int QMV_LDS_BUDGET = 64 * 1024;

template <int T, int M, bool DUMP>
static int launch_qmv_t(const uint8_t* W, int N, int K, const uint8_t* xq, float* y,
                        int32_t* isums, hipStream_t s) {
  constexpr int R = QmvCfg<M>::R;
  // K-chunk: multiple of 256 that fits the LDS budget, chunks of equal size.
  const int per_k = M + M * 16 / Q8_BLOCK;  // bytes of LDS per activation column
  const int red_bytes = QMV_WAVES * QMV_SLOTS * R * M * (int)sizeof(double);
  int kcmax = ((QMV_LDS_BUDGET - red_bytes) / per_k) / QK * QK;
  if (kcmax < QK) kcmax = QK;
  const int nsb = K / QK;
  const int nchunk = (K + kcmax - 1) / kcmax;
  const int kc = ((nsb + nchunk - 1) / nchunk) * QK;
  const size_t lds = (size_t)M * kc + (size_t)M * (kc / Q8_BLOCK) * sizeof(DsEntry) + red_bytes;
  if (lds > (size_t)QMV_LDS_BUDGET) return -1;
  const int rows_per_wg = QMV_SLOTS * R;
  const int grid = (N + rows_per_wg - 1) / rows_per_wg;
  hipLaunchKernelGGL((qmv_dot4_kernel<T, M, R, DUMP>), dim3(grid), dim3(QMV_THREADS), lds, s, W, N,
                     K, xq, y, isums, kc);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int T, bool DUMP>
static int launch_qmv_m(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                        int32_t* isums, hipStream_t s) {
  switch (M) {
    case 1: return launch_qmv_t<T, 1, DUMP>(W, N, K, xq, y, isums, s);
    case 2: return launch_qmv_t<T, 2, DUMP>(W, N, K, xq, y, isums, s);
    case 3: return launch_qmv_t<T, 3, DUMP>(W, N, K, xq, y, isums, s);
    case 4: return launch_qmv_t<T, 4, DUMP>(W, N, K, xq, y, isums, s);
    case 5: return launch_qmv_t<T, 5, DUMP>(W, N, K, xq, y, isums, s);
    case 6: return launch_qmv_t<T, 6, DUMP>(W, N, K, xq, y, isums, s);
    case 7: return launch_qmv_t<T, 7, DUMP>(W, N, K, xq, y, isums, s);
    case 8: return launch_qmv_t<T, 8, DUMP>(W, N, K, xq, y, isums, s);
    default: return -2;
  }
}

int launch_qmv(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s) {
  const uint8_t* w8 = static_cast<const uint8_t*>(W);
  const uint8_t* x8 = static_cast<const uint8_t*>(xq);
  const bool dump = isums != nullptr;
  switch (type) {
    case Q4_K:
      return dump ? launch_qmv_m<Q4_K, true>(w8, N, K, x8, M, y, isums, s)
                  : launch_qmv_m<Q4_K, false>(w8, N, K, x8, M, y, isums, s);
    case Q6_K:
      return dump ? launch_qmv_m<Q6_K, true>(w8, N, K, x8, M, y, isums, s)
                  : launch_qmv_m<Q6_K, false>(w8, N, K, x8, M, y, isums, s);
    case IQ4_XS:
      return dump ? launch_qmv_m<IQ4_XS, true>(w8, N, K, x8, M, y, isums, s)
                  : launch_qmv_m<IQ4_XS, false>(w8, N, K, x8, M, y, isums, s);
    default:
      return -2;
  }
}

}  // namespace qdot
