// qmv_kernel.hpp -- decode matmul for M = 1..8 token rows, and for Q4_K and
// IQ4_XS up to 16 (rows a2-a5 of the hot path): y[m][n] = sum_k w[n][k] *
// xhat[m][k] on the raw Q4_K / Q6_K / IQ4_XS superblocks, with v_dot4_i32_i8
// or MFMA i8 integer dots against Q8_1 activations.
//
// What the pages fix, and what this kernel keeps:
//  * integer dots on the raw quantized weights, fp32 out, no fp32 weight copy
//    (xLLM v0.7 log, section 1);
//  * an M-row tile, so each weight byte is read from HBM once for all M rows
//    (xLLM section B2, q4k_dp4a_matmul_q8_v2_kernel<M>; V100TPS 2026-08-12:
//    the batched matvec reads the weights once for all token positions);
//  * the weight decode and the IQ4_NL lookup done once per weight, not once per
//    row (V100TPS 2026-08-12: moving the kvalues lookup to load time gave 1.5x);
//  * exact int32 sums inside each sub-block, scales applied afterwards
//    (Kestrel section 5).
// What differs from the pages' V100 design: the M=8 V100 kernel was L1-bound
// (xLLM section B2 ncu table).  Here each wave of a workgroup takes every
// P-th superblock of 16 weight rows (4 lanes per row, 64 weights per lane);
// the activations of a superblock (8*M Q8_1 blocks) are fetched one block per
// lane together with its weights and published to the wave's LDS slice just
// before use, so the 16 rows of the wave read them as LDS broadcasts instead
// of pulling them through the vector memory path once per row.  The scale
// drains are exact fp64 terms (every product exact, one rounding per
// accumulate), so y is the fp32 rounding of a value within a few fp64 ulps
// of the exact sum.

#pragma once

#include <type_traits>

#include "formats.hpp"

namespace qdot {

constexpr int QMV_MAX_THREADS = 512;  // up to 8 waves per workgroup
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

// Q4_0: eight 18-byte blocks {fp16 d, qs[16]} per 256-weight group; quarter
// q = blocks 2q and 2q+1 = bytes 36q .. 36q+35 (2-byte aligned fields).
template <> struct Fmt<Q4_0> {
  struct Regs { u32x4 a, b; uint32_t c; };
  __device__ static Regs load(const uint8_t* sb, int q) {
    Regs r;
    r.a = ld16(sb + 36 * q);
    r.b = ld16(sb + 36 * q + 16);
    r.c = ld4(sb + 36 * q + 32);
    return r;
  }
  __device__ static int blk(int q, int half) { return 2 * q + half; }
};

// Q8_0: eight 34-byte blocks {fp16 d, int8 qs[32]} per group; quarter q =
// blocks 2q and 2q+1 = bytes 68q .. 68q+67.
template <> struct Fmt<Q8_0> {
  struct Regs { u32x4 a, b, c, e; uint32_t f; };
  __device__ static Regs load(const uint8_t* sb, int q) {
    Regs r;
    r.a = ld16(sb + 68 * q);
    r.b = ld16(sb + 68 * q + 16);
    r.c = ld16(sb + 68 * q + 32);
    r.e = ld16(sb + 68 * q + 48);
    r.f = ld4(sb + 68 * q + 64);
    return r;
  }
  __device__ static int blk(int q, int half) { return 2 * q + half; }
};

// ---------------------------------------------------------------- kernels
//
// One lane handles quarter q of superblock b for one weight row (slot s, row
// n0 + s).  The P waves of a workgroup split the superblocks of each row:
// wave w takes b = w, w+P, ...  P is a function of K only, and the kernel
// walks a lane's superblocks and halves in the same order with the same fp64
// operations for every M, so row m of y does not depend on M.

// Per-row, per-half-quarter weight data: the 8 code dwords (32 int8 codes in
// activation order) and what the drain needs.
template <int T> struct Sub;
template <> struct Sub<Q4_K> { uint32_t cw[8]; double wsc, wmn; };
template <> struct Sub<IQ4_XS> { uint32_t cw[8]; double wsc; };
template <> struct Sub<Q6_K> { uint32_t cw[8]; int s0, s1; double d; };
template <> struct Sub<Q4_0> { uint32_t cw[8]; double wsc; };
template <> struct Sub<Q8_0> { uint32_t cw[8]; double wsc; };

template <int T>
__device__ __forceinline__ void decode_sub(const typename Fmt<T>::Regs& g, int q, int half,
                                           Sub<T>& o) {
  if constexpr (T == Q4_K) {
    q4k_scales(g.h, 2 * q + half, o.wsc, o.wmn);       // sub-block 2q + half
    const uint32_t pk[8] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o.cw[i] = (half ? (pk[i] >> 4) : pk[i]) & 0x0F0F0F0Fu;
  } else if constexpr (T == IQ4_XS) {
    o.wsc = iq4xs_scale(g.h.x, g.h.y, 2 * q + half);
    const u32x4 pq = half ? g.b : g.a;
    const uint32_t pk[4] = {pq.x, pq.y, pq.z, pq.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o.cw[i] = iq4nl_lookup(pk[i]);           // elements 4i..4i+3
      o.cw[i + 4] = iq4nl_lookup(pk[i] >> 4);  // elements 16+4i..
    }
  } else if constexpr (T == Q4_0) {
    // block 2q (bytes 0-17) or 2q+1 (bytes 18-35); raw nibbles 0..15, the -8
    // offset is applied through the activation block sum
    const uint32_t w[9] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w, g.c};
    uint32_t qs[4];
    if (half == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i] = shr16(w[i + 1], w[i]);
      o.wsc = (double)h2f(w[0]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qs[i] = w[5 + i];
      o.wsc = (double)h2f(w[4] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o.cw[i] = qs[i] & 0x0F0F0F0Fu;             // elements 4i..4i+3
      o.cw[i + 4] = (qs[i] >> 4) & 0x0F0F0F0Fu;  // elements 16+4i..
    }
  } else if constexpr (T == Q8_0) {
    const uint32_t w[17] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w,
                            g.c.x, g.c.y, g.c.z, g.c.w, g.e.x, g.e.y, g.e.z, g.e.w, g.f};
    if (half == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) o.cw[i] = shr16(w[i + 1], w[i]);
      o.wsc = (double)h2f(w[0]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) o.cw[i] = w[9 + i];
      o.wsc = (double)h2f(w[8] >> 16);
    }
  } else {  // Q6_K
    const int h = q >> 1, gp = q & 1;
    // codes of Q8 block 4h+gp (half 0: g = gp, low nibbles) or 4h+gp+2 (half
    // 1: g = gp+2, high nibbles): values 0..63; the -32 offset is applied
    // through the activation half-sums.
    const uint32_t pl[8] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y, g.b.z, g.b.w};
    const uint32_t ph[8] = {g.c.x, g.c.y, g.c.z, g.c.w, g.e.x, g.e.y, g.e.z, g.e.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) o.cw[i] = half ? q6k_code<1>(pl[i], ph[i], gp) : q6k_code<0>(pl[i], ph[i], gp);
    // int8 sub-scales of sub-blocks t0 = 8h + 2gp + 4*half and t0 + 1
    const uint32_t scw = h ? (half ? g.sc.w : g.sc.z) : (half ? g.sc.y : g.sc.x);
    o.s0 = (int)(int8_t)(scw >> (16 * gp));
    o.s1 = (int)(int8_t)(scw >> (16 * gp + 8));
    o.d = (double)h2f(g.d);
  }
}

// Index of the first sub-block (of length SUB) that (q, half) covers inside
// its superblock; Q6_K covers two consecutive 16-element sub-blocks.
template <int T> __device__ __forceinline__ int sub_index(int q, int half) {
  if constexpr (T == Q6_K) return 8 * (q >> 1) + 2 * (q & 1) + 4 * half;
  else return 2 * q + half;
}

// fp64 view of one Q8_1 block's scales: D and (Q4_K) S, or (Q6_K) 32 times
// the integer sum of each 16-element half of q (for the -32 code offset), or
// (Q4_0) 8 times the integer sum of q (for the -8 code offset).
// The same from the block's d | s << 16 bits and the code sums of its two
// 16-element halves.
__device__ __forceinline__ DsEntry ds_entry_sums(int T, uint32_t ds, int lo, int hi) {
  DsEntry e;
  e.d = (double)h2f(ds & 0xFFFFu);
  if (T == Q4_0) {
    e.xs32[0] = 8 * (lo + hi);
    e.xs32[1] = 0;
  } else if (T == Q6_K) {
    e.xs32[0] = 32 * lo;
    e.xs32[1] = 32 * hi;
  } else {
    e.s = (double)h2f(ds >> 16);
  }
  return e;
}
__device__ __forceinline__ DsEntry ds_entry(int T, uint32_t ds, const u32x4& q0, const u32x4& q1) {
  if (T != Q4_0 && T != Q6_K) return ds_entry_sums(T, ds, 0, 0);
  const uint32_t ones = 0x01010101u;
  const int lo = dot4(q0.w, ones, dot4(q0.z, ones, dot4(q0.y, ones, dot4(q0.x, ones, 0))));
  const int hi = dot4(q1.w, ones, dot4(q1.z, ones, dot4(q1.y, ones, dot4(q1.x, ones, 0))));
  return ds_entry_sums(T, ds, lo, hi);
}

// The integer dots of one (row, activation row, half quarter) and their
// exact-term fp64 drain into acc.  Optionally stores the int32 sums.
template <int T, bool DUMP>
__device__ __forceinline__ void dot_drain(const Sub<T>& sw, const uint32_t (&xa)[8],
                                          const DsEntry& de, double& acc, int32_t* isp) {
  if constexpr (T == Q6_K) {
    int I0 = 0, I1 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) I0 = dot4(sw.cw[i], xa[i], I0);
#pragma unroll
    for (int i = 4; i < 8; ++i) I1 = dot4(sw.cw[i], xa[i], I1);
    I0 -= de.xs32[0];
    I1 -= de.xs32[1];
    const int Pq = q6k_pair(sw.s0, I0, sw.s1, I1);        // exact int
    acc = fma(sw.d * de.d, (double)Pq, acc);              // exact product, one rounding
    if (DUMP && isp) { isp[0] = I0; isp[1] = I1; }
  } else {
    int I = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) I = dot4(sw.cw[i], xa[i], I);
    if constexpr (T == Q4_0) I -= de.xs32[0];             // sum (q - 8) x
    acc = fma(sw.wsc * de.d, (double)I, acc);             // exact product, one rounding
    if constexpr (T == Q4_K) acc = fma(sw.wmn, de.s, acc);
    if (DUMP && isp) isp[0] = I;
  }
}

template <int T, int M, int R, bool DUMP>
__device__ __forceinline__ int32_t* isum_ptr(int32_t* isums, int N, int K, int m, int n, int b, int q,
                                             int half) {
  constexpr int SUB = Geom<T>::SUB;
  if (!DUMP || n >= N) return nullptr;
  return isums + ((size_t)m * N + n) * (K / SUB) + (size_t)b * (QK / SUB) + sub_index<T>(q, half);
}

// Quad reduction (the 4 quarter lanes of a slot), then over the P waves in
// order through LDS, then the fp32 store.  lds_red holds P*16*R*M doubles.
template <int M, int R>
__device__ __forceinline__ void reduce_store(double (&acc)[R][M], double* lds_red, int P, int wave,
                                             int slot, int q, int tid, int n0, int N,
                                             float* __restrict__ y) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) {
      double v = acc[r][m];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      acc[r][m] = v;
    }
  __syncthreads();  // the staging area is reused for the reduction
  if (q == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m)
        lds_red[((wave * QMV_SLOTS + slot) * R + r) * M + m] = acc[r][m];
  }
  __syncthreads();
  for (int o = tid; o < QMV_SLOTS * R * M; o += 64 * P) {
    const int m = o % M;
    const int r = (o / M) % R;
    const int s = o / (M * R);
    const int n = n0 + s + QMV_SLOTS * r;
    double v = lds_red[(s * R + r) * M + m];
    for (int w = 1; w < P; ++w) v += lds_red[((w * QMV_SLOTS + s) * R + r) * M + m];
    if (n < N) y[(size_t)m * N + n] = (float)v;
  }
}

// ------------------------------------------------------ the decode kernel
constexpr int QMV_MGROUP = 4;  // activation rows held in registers at once

// Each wave stages the activations of its own superblocks: for superblock b
// the 8*M Q8_1 blocks (M rows x 8 blocks) are loaded one per lane, together
// with the weights of b, and written to the wave's LDS slice just before b
// is computed.  A load's data is waited for only when its superblock comes
// up, so no wait covers weights fetched for later superblocks, and no
// workgroup barrier sits in the main loop.
// The work of one workgroup: weight rows 16*tile .. 16*tile+15 of one matrix.
//
// XF: the activations arrive as fp32 rows x [M][K] (xq points at them) and
// each wave quantizes the 8*M Q8_1 blocks of its superblock itself, into the
// same LDS slice, with the standalone quantizer's code (q8_1_block8), so the
// slice holds the same bytes quantize_q8_1 would have written: one launch
// instead of a quantize launch and a matmul launch, and bitwise the same y.
template <int T, int M, int DEPTH, bool DUMP, bool XF = false>
__device__ __forceinline__ void qmv_tile(const uint8_t* __restrict__ W, int N, int K,
                                         const uint8_t* __restrict__ xq, float* __restrict__ y,
                                         int32_t* __restrict__ isums, int tile, uint8_t* smem) {
  static_assert(!(XF && DUMP), "the sub-block dump reads quantized activations");
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int ITEMS = 8 * M;  // Q8_1 blocks per superblock and activation rows
  static_assert(ITEMS <= 64, "one activation block per lane");
  const int P = blockDim.x >> 6;
  const int nsb = K / QK;
  const int nq8 = K / Q8_BLOCK;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, slot = lane >> 2, q = lane & 3;
  const int n0 = tile * QMV_SLOTS;

  // this wave's LDS slice: codes [M][8][32 B], then scales [M][8]
  uint8_t* lds_x = smem + (size_t)wave * ITEMS * (Q8_BLOCK + sizeof(DsEntry));
  DsEntry* lds_ds = reinterpret_cast<DsEntry*>(lds_x + ITEMS * Q8_BLOCK);

  const int nrow = n0 + slot;
  const uint8_t* wrow = W + (size_t)(nrow < N ? nrow : N - 1) * nsb * BYTES;
  // activation block of this lane: item = m*8 + j (lanes past 8*M repeat one)
  const int item = lane % ITEMS;
  const uint8_t* xsrc = xq + ((size_t)(item >> 3) * nq8 + (item & 7)) * Q8_BYTES;

  double acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0;

  // XF: this lane's four fp32 values of block j = lane / 8 of the superblock
  // (part lane % 8), for each activation row
  const uint8_t* xfsrc = xq + (size_t)(32 * (lane >> 3) + 4 * (lane & 7)) * sizeof(float);

  struct XStage { uint32_t ds; u32x4 c0, c1; };   // one Q8_1 block
  struct FStage { u32x4 v[M]; };                   // fp32 values, one row each
  struct Stage {
    typename Fmt<T>::Regs w;
    typename std::conditional<XF, FStage, XStage>::type x;
  };
  Stage S[DEPTH];
  // Unconditional loads (superblock clamped to the row): the compiler then
  // waits for exactly the stage a compute step uses.
  auto fetch = [&](Stage& st, int bsb) {
    const int bc = bsb < nsb ? bsb : nsb - 1;
    st.w = Fmt<T>::load(wrow + (size_t)bc * BYTES, q);
    if constexpr (XF) {
#pragma unroll
      for (int m = 0; m < M; ++m)
        st.x.v[m] = ld16(xfsrc + ((size_t)m * K + (size_t)bc * QK) * sizeof(float));
    } else {
      const uint8_t* src = xsrc + (size_t)bc * 8 * Q8_BYTES;
      st.x.ds = ld4(src);
      st.x.c0 = ld16(src + 4);
      st.x.c1 = ld16(src + 20);
    }
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto compute = [&](const Stage& st, int b) {
    wave_sync();  // the previous superblock's LDS reads are done
    if constexpr (XF) {
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v[4] = {__uint_as_float(st.x.v[m].x), __uint_as_float(st.x.v[m].y),
                            __uint_as_float(st.x.v[m].z), __uint_as_float(st.x.v[m].w)};
        uint32_t packed, ds;
        int part_sum, sumq;
        q8_1_block8(v, packed, part_sum, sumq, ds);
        // code sums of the block's halves (parts 0-3, 4-7) for the -32 / -8 offsets
        int h = part_sum;
        h += __shfl_xor(h, 1);
        h += __shfl_xor(h, 2);
        const int hi = __shfl_xor(h, 4);
        const int it = 8 * m + (lane >> 3);
        *reinterpret_cast<uint32_t*>(lds_x + it * Q8_BLOCK + 4 * (lane & 7)) = packed;
        if ((lane & 7) == 0) lds_ds[it] = ds_entry_sums(T, ds, h, hi);
      }
    } else {
      if (lane < ITEMS) {
        *reinterpret_cast<u32x4*>(lds_x + item * Q8_BLOCK) = st.x.c0;
        *reinterpret_cast<u32x4*>(lds_x + item * Q8_BLOCK + 16) = st.x.c1;
        lds_ds[item] = ds_entry(T, st.x.ds, st.x.c0, st.x.c1);
      }
    }
    wave_sync();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kb = Fmt<T>::blk(q, half);  // Q8_1 block within the superblock
      Sub<T> sw;
      decode_sub<T>(st.w, q, half, sw);
#pragma unroll
      for (int m0 = 0; m0 < M; m0 += QMV_MGROUP) {
        constexpr int G = QMV_MGROUP;
        uint32_t xa[G][8];
        DsEntry de[G];
#pragma unroll
        for (int mm = 0; mm < G; ++mm) {
          if (m0 + mm < M) {
            const int it = (m0 + mm) * 8 + kb;
            const u32x4 v0 = *reinterpret_cast<const u32x4*>(lds_x + it * Q8_BLOCK);
            const u32x4 v1 = *reinterpret_cast<const u32x4*>(lds_x + it * Q8_BLOCK + 16);
            xa[mm][0] = v0.x; xa[mm][1] = v0.y; xa[mm][2] = v0.z; xa[mm][3] = v0.w;
            xa[mm][4] = v1.x; xa[mm][5] = v1.y; xa[mm][6] = v1.z; xa[mm][7] = v1.w;
            de[mm] = lds_ds[it];
          }
        }
#pragma unroll
        for (int mm = 0; mm < G; ++mm)
          if (m0 + mm < M)
            dot_drain<T, DUMP>(sw, xa[mm], de[mm], acc[m0 + mm],
                               isum_ptr<T, M, 1, DUMP>(isums, N, K, m0 + mm, nrow, b, q, half));
      }
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(S[d], wave + d * P);
  const int niter = (((nsb + P - 1) / P) + DEPTH - 1) / DEPTH * DEPTH;
  auto step = [&](Stage& st, int ii, bool refill) {
    const int b = wave + ii * P;
    if (b < nsb) compute(st, b);
    if (refill) fetch(st, b + DEPTH * P);
  };
  // The last DEPTH iterations are peeled so that no prefetch runs past the
  // row (a redundant load would still have to land before the wave retires).
  int i = 0;
  for (; i + DEPTH < niter; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, true);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, false);

  double acc2[1][M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc2[0][m] = acc[m];
  reduce_store<M, 1>(acc2, reinterpret_cast<double*>(smem), P, wave, slot, q, tid, n0, N, y);
}

// ------------------------------------------ Q6_K on 16 x 16 MFMA tiles
//
// Q6_K at M >= Q6F_MIN_M: the same workgroup (16 weight rows), K split,
// activation staging and summation order as qmv_tile, but the integer dots
// come from one v_mfma_i32_16x16x32_i8 per Q8_1 block.  At M = 8 qmv_tile's
// 16 row slots each read all 8*M staged activation blocks of a superblock
// from LDS; here a lane reads 8 bytes per block.
//
// Lane l (c16 = l % 16, g4 = l / 16) supplies B = the signed codes of weight
// row c16, elements 8*g4 .. 8*g4+7 of the block, and A row c16, which holds
// activation row c16 / 2 in "slot" c16 % 2: slot 0 carries elements 0-15 of
// the block (the first 16-element sub-block) and zeros for 16-31, slot 1 the
// reverse, so one MFMA gives both sub-block sums.  Result v of lane l is
// D[4*g4 + v][c16] (gfx950 layout): the sums I0 (v = 2k) and I1 (v = 2k+1)
// of activation row 2*g4 + k.  The lane drains d*D*(s0*I0 + s1*I1) -- the
// same exact integer and the same fp64 fma as qmv_tile (whose -32 code
// offset goes through the activation sums instead) -- into per-quarter
// accumulators in qmv_tile's block order, then adds the quarters as
// qmv_tile's quad reduction does, and the waves are added in order: every
// output is bitwise qmv_tile's.
constexpr int Q6F_MIN_M = 7;
template <int T, int M> constexpr bool q6f_ok() { return T == Q6_K && M >= Q6F_MIN_M && M <= 8; }

template <int M, int DEPTH, bool DUMP>
__device__ __forceinline__ void q6f_tile(const uint8_t* __restrict__ W, int N, int K,
                                         const uint8_t* __restrict__ xq, float* __restrict__ y,
                                         int32_t* __restrict__ isums, int tile, uint8_t* smem) {
  typedef int v4i_q __attribute__((ext_vector_type(4)));
  constexpr int BYTES = Geom<Q6_K>::BYTES;
  constexpr int ITEMS = 8 * M;
  const int P = blockDim.x >> 6;
  const int nsb = K / QK;
  const int nq8 = K / Q8_BLOCK;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int n0 = tile * QMV_SLOTS;

  // the wave's LDS slice (qmv_tile's size): the codes of activation row m at
  // m * Q6F_APITCH (the 32 distinct 8-byte A reads of a block on distinct
  // banks; a 256-byte row pitch would put all eight rows on the same ones),
  // then the fp64 D of each block
  constexpr int Q6F_APITCH = 8 * Q8_BLOCK + 32;
  static_assert(M * Q6F_APITCH + ITEMS * 8 <= ITEMS * (Q8_BLOCK + (int)sizeof(DsEntry)), "slice size");
  uint8_t* lds_x = smem + (size_t)wave * ITEMS * (Q8_BLOCK + sizeof(DsEntry));
  double* lds_d = reinterpret_cast<double*>(lds_x + M * Q6F_APITCH);

  const int nrow = n0 + c16;
  const uint8_t* wrow = W + (size_t)(nrow < N ? nrow : N - 1) * nsb * BYTES;
  const int item = lane % ITEMS;
  const uint8_t* xsrc = xq + ((size_t)(item >> 3) * nq8 + (item & 7)) * Q8_BYTES;
  // A row of this lane: activation row am = c16 / 2 in slot c16 % 2; zero
  // where the lane's K-slice is not in its slot's sub-block or am >= M
  const int am = c16 >> 1;
  const bool a_on = (g4 >> 1) == (c16 & 1) && am < M;
  const uint8_t* a_src = lds_x + (size_t)(am < M ? am : 0) * Q6F_APITCH + 8 * g4;

  // activation rows 2*g4 + k (k = 0, 1) of this lane's results (clamped into
  // the staged rows; rows >= M are never stored)
  int dm[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) dm[k] = 2 * g4 + k < M ? 2 * g4 + k : 0;

  double acc[4][2];  // [quarter][k]
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int k = 0; k < 2; ++k) acc[q][k] = 0.0;

  // weights: K-slice g4 of every block of the row -- ql bytes 8*g4 .. +7 of
  // each 32-byte run of both halves, qh bytes 8*g4 .. +7 of each half --
  // plus the sub-scales and d; activations: one Q8_1 block per lane, as qmv_tile
  struct Stage { u32x2 l0[2], l1[2], qh[2]; u32x4 sc; uint32_t d; uint32_t ds; u32x4 c0, c1; };
  Stage S[DEPTH];
  auto fetch = [&](Stage& st, int bsb) {
    const int bc = bsb < nsb ? bsb : nsb - 1;
    const uint8_t* sb = wrow + (size_t)bc * BYTES;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      st.l0[h] = ld8(sb + 64 * h + 8 * g4);
      st.l1[h] = ld8(sb + 64 * h + 32 + 8 * g4);
      st.qh[h] = ld8(sb + 128 + 32 * h + 8 * g4);
    }
    st.sc = ld16(sb + 192);
    unsigned short dh;
    __builtin_memcpy(&dh, sb + 208, 2);
    st.d = dh;
    const uint8_t* src = xsrc + (size_t)bc * 8 * Q8_BYTES;
    st.ds = ld4(src);
    st.c0 = ld16(src + 4);
    st.c1 = ld16(src + 20);
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto compute = [&](const Stage& st, int b) {
    wave_sync();  // the previous superblock's LDS reads are done
    if (lane < ITEMS) {
      uint8_t* dst = lds_x + (item >> 3) * Q6F_APITCH + (item & 7) * Q8_BLOCK;
      *reinterpret_cast<u32x4*>(dst) = st.c0;
      *reinterpret_cast<u32x4*>(dst + 16) = st.c1;
      lds_d[item] = (double)h2f(st.ds & 0xFFFFu);
    }
    wave_sync();
    const double dw = (double)h2f(st.d);
    // all eight blocks' MFMAs first, then the drains; no branch splits the
    // superblock (rows >= M drain clamped copies that are never stored)
    v4i_q I[8];
    auto mfma_block = [&](auto JC) {
      constexpr int J = decltype(JC)::value;
      constexpr int h = J >> 2, g6 = J & 3;
      const u32x2 src = (g6 & 1) ? st.l1[h] : st.l0[h];
      const uint32_t bx = q6k_signed(q6k_code<(g6 >= 2)>(src.x, st.qh[h].x, g6 & 1));
      const uint32_t by = q6k_signed(q6k_code<(g6 >= 2)>(src.y, st.qh[h].y, g6 & 1));
      const long bq = (long)((uint64_t)bx | ((uint64_t)by << 32));
      const u32x2 av = *reinterpret_cast<const u32x2*>(a_src + J * Q8_BLOCK);
      const long aq = a_on ? (long)((uint64_t)av.x | ((uint64_t)av.y << 32)) : 0L;
      const v4i_q z = {0, 0, 0, 0};
      I[J] = __builtin_amdgcn_mfma_i32_16x16x32_i8(aq, bq, z, 0, 0, 0);
    };
    auto drain_block = [&](auto JC) {
      constexpr int J = decltype(JC)::value;
      constexpr int q = 2 * (J >> 2) + (J & 1);  // qmv_tile's quarter of block J
      const uint32_t scw = (J < 2 ? st.sc.x : (J < 4 ? st.sc.y : (J < 6 ? st.sc.z : st.sc.w))) >> (16 * (J & 1));
      const int s0 = (int)(int8_t)scw, s1 = (int)(int8_t)(scw >> 8);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int I0 = I[J][2 * k], I1 = I[J][2 * k + 1];  // sub-blocks 2J, 2J+1 of row 2*g4 + k
        const int Pq = q6k_pair(s0, I0, s1, I1);  // exact int
        acc[q][k] = fma(dw * lds_d[dm[k] * 8 + J], (double)Pq, acc[q][k]);
        if (DUMP && 2 * g4 + k < M && nrow < N) {
          int32_t* p = isums + ((size_t)(2 * g4 + k) * N + nrow) * (K / 16) + (size_t)b * 16 + 2 * J;
          p[0] = I0;
          p[1] = I1;
        }
      }
    };
    mfma_block(std::integral_constant<int, 0>{});
    mfma_block(std::integral_constant<int, 1>{});
    mfma_block(std::integral_constant<int, 2>{});
    mfma_block(std::integral_constant<int, 3>{});
    mfma_block(std::integral_constant<int, 4>{});
    mfma_block(std::integral_constant<int, 5>{});
    mfma_block(std::integral_constant<int, 6>{});
    mfma_block(std::integral_constant<int, 7>{});
    drain_block(std::integral_constant<int, 0>{});
    drain_block(std::integral_constant<int, 1>{});
    drain_block(std::integral_constant<int, 2>{});
    drain_block(std::integral_constant<int, 3>{});
    drain_block(std::integral_constant<int, 4>{});
    drain_block(std::integral_constant<int, 5>{});
    drain_block(std::integral_constant<int, 6>{});
    drain_block(std::integral_constant<int, 7>{});
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(S[d], wave + d * P);
  const int niter = (((nsb + P - 1) / P) + DEPTH - 1) / DEPTH * DEPTH;
  auto step = [&](Stage& st, int ii, bool refill) {
    const int b = wave + ii * P;
    if (b < nsb) compute(st, b);
    if (refill) fetch(st, b + DEPTH * P);
  };
  int i = 0;
  for (; i + DEPTH < niter; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, true);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, false);

  // quarters as qmv_tile's quad reduction adds them, then the waves in order
  __syncthreads();  // the staging area is reused for the reduction
  double* red = reinterpret_cast<double*>(smem);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int m = 2 * g4 + k;
    if (m < M) red[(wave * QMV_SLOTS + c16) * M + m] = (acc[0][k] + acc[1][k]) + (acc[2][k] + acc[3][k]);
  }
  __syncthreads();
  for (int o = tid; o < QMV_SLOTS * M; o += 64 * P) {
    const int m = o % M, sl = o / M;
    const int n = n0 + sl;
    double v = red[sl * M + m];
    for (int w = 1; w < P; ++w) v += red[(w * QMV_SLOTS + sl) * M + m];
    if (n < N) y[(size_t)m * N + n] = (float)v;
  }
}

// ------------------------------------------ the MFMA tile for M = 7, 8
//
// The same sums as qmv_tile, in the same fp64 order, with the integer dots
// on v_mfma_i32_32x32x32_i8 (Q4_K and IQ4_XS weights: 32-element sub-blocks,
// two per quarter, like the dot4 tile's).  At M = 8 each of qmv_tile's 16
// row slots reads all 8*M activation blocks of a superblock from LDS (48 KB
// per wave and superblock); here the matrix unit reuses every activation byte
// across 32 weight rows, and only the fp64 scales go through LDS.
//
// A workgroup owns 32 weight rows; its P waves split K exactly as qmv_tile's
// (wave w takes superblocks w, w+P, ...).  Lane l supplies weight row
// n = l%32 (B operand: 16 codes of K-slice s = l/32) and row i = l%32 of the
// A operand, which holds activation row m = i%8 of the Q8_1 block in "slot"
// i/8: the 32-row A tile stacks the four blocks of a group (sub-blocks 4g ..
// 4g+3, i.e. quarters 2g and 2g+1) for 8 activation rows, and the MFMA of
// sub-block 4g+j zeroes the other slots' rows, so after the group's four
// MFMAs result register r of lane l holds the exact int32 sum of activation
// row 4s + r%4, weight row n and sub-block 4g + r/4 (gfx950 layout:
// D[8(r/4) + 4s + r%4][l%32]).  Lane l then drains its 4 activation rows into
// per-quarter fp64 accumulators in qmv_tile's order (sub-block 2q before
// 2q+1, superblocks in wave order), and the quarters and waves are added in
// qmv_tile's order, so every output is bitwise the same as qmv_tile's: rows
// stay M-invariant across the two tiles.
typedef int qmf_v4i __attribute__((ext_vector_type(4)));
typedef int qmf_v16i __attribute__((ext_vector_type(16)));

constexpr int QMF_ROWS = 32;  // weight rows per workgroup
// Which Q4_K launches take the MFMA tile (measured on MI355X, Qwen3-8B
// shapes).  Alone (qdot_qmatmul): M >= 7 -- a 4096 x 4096 launch is faster
// on the dot4 tile up to M = 6, its 128 MFMA workgroups being too few.  In a
// grouped launch (qdot_qmatmul_multi) the launcher decides per launch (MF):
// q+k+v (K = 4096) is faster on MFMA tiles at every M (M = 1: 7.2 vs 7.9 us,
// M = 4: 8.1 vs 9.9), gate+up from M = 3; at K = 1536 (Qwen2.5-1.5B) the dot4
// tile stays faster.  Either tile gives bitwise the same rows.
// IQ4_XS (hidden-5120 shapes): its dot4 tile looks the codebook up for every
// weight, so the MFMA tile wins from M = 5 (5120 x 7168 at M = 7: 10.9 vs
// 14.5 us; at M = 4 the dot4 tile: 10.2 vs 10.8).
template <int T> constexpr bool qmf_type() { return T == Q4_K || T == IQ4_XS; }
template <int T> constexpr int qmf_min_m() { return T == IQ4_XS ? 5 : 7; }
template <int T, int M> constexpr bool qmf_ok() { return qmf_type<T>() && M >= qmf_min_m<T>(); }
template <int T, int M, bool MF> constexpr bool qmf_group_ok() { return MF && qmf_type<T>(); }
template <int T, int M> constexpr int qmv_tile_rows() { return qmf_ok<T, M>() ? QMF_ROWS : QMV_SLOTS; }

struct __attribute__((aligned(16))) QmfDs { double d, s; };  // fp64 D and S of one Q8_1 block

// The MFMA tile also takes M = 9..16 (Q4_K and IQ4_XS, through qdot_qmatmul):
// 16 activation rows per A-tile slot instead of 8, two sub-blocks per group.
constexpr int QMF_MAX_M = 16;
template <int M> constexpr int qmf_rows() { return M <= 8 ? 8 : 16; }

template <int T, int M, int DEPTH, bool DUMP>
__device__ __forceinline__ void qmf_tile(const uint8_t* __restrict__ W, int N, int K,
                                         const uint8_t* __restrict__ xq, float* __restrict__ y,
                                         int32_t* __restrict__ isums, int tile, uint8_t* smem) {
  static_assert(qmf_type<T>(), "the MFMA decode tile takes Q4_K or IQ4_XS weights");
  constexpr int NQ = T == Q4_K ? 4 : 8;  // 16-byte code loads per superblock and lane
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int SUB = Geom<T>::SUB;
  const int P = blockDim.x >> 6;
  const int nsb = K / QK;
  const int nq8 = K / Q8_BLOCK;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, s = lane >> 5;
  const int slot = (lane & 31) >> 3, mrow = lane & 7;  // this lane's A row: block slot, activation row
  const int n0 = tile * QMF_ROWS;
  const int nrow = n0 + n;
  const uint8_t* wrow = W + (size_t)(nrow < N ? nrow : N - 1) * nsb * BYTES;
  // this lane's A data: row mrow (rows >= M read row 0 and are masked to zero)
  const uint8_t* xa_row = xq + ((size_t)(mrow < M ? mrow : 0) * nq8 + slot) * Q8_BYTES + 4 + 16 * s;
  const uint32_t amask = mrow < M ? 0xFFFFFFFFu : 0u;
  // scale entry this lane publishes per superblock: activation row lane/8, block lane%8
  const int dm = lane >> 3, dj = lane & 7;
  const uint8_t* xd_src = xq + ((size_t)(dm < M ? dm : 0) * nq8 + dj) * Q8_BYTES;
  QmfDs* lds_ds = reinterpret_cast<QmfDs*>(smem) + wave * 64;

  double acc[4][4];  // [quarter][activation row 4s + mm]
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) acc[q][mm] = 0.0;

  // Q4_K: header (d, dmin, scales) and the code bytes of K-slice s of each
  // quarter (low nibbles sub-block 2q, high 2q+1).  IQ4_XS: header (d,
  // scales_h, scales_l) and the 16 code bytes of each sub-block (low nibbles
  // its elements 0-15 = K-slice 0, high nibbles 16-31 = K-slice 1).
  struct Stage {
    u32x4 h, q[NQ];
    u32x4 a[2];     // this lane's A data in groups 0 and 1
    uint32_t ds;    // d, s of the published scale entry
  };
  Stage S[DEPTH];
  auto fetch = [&](Stage& st, int bsb) {
    const int bc = bsb < nsb ? bsb : nsb - 1;
    const uint8_t* sb = wrow + (size_t)bc * BYTES;
    st.h = ld16(sb);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      st.q[q] = T == Q4_K ? ld16(sb + 16 + 32 * q + 16 * s) : ld16(sb + 8 + 16 * q);
#pragma unroll
    for (int g = 0; g < 2; ++g) st.a[g] = ld16(xa_row + (size_t)(8 * bc + 4 * g) * Q8_BYTES);
    st.ds = ld4(xd_src + (size_t)8 * bc * Q8_BYTES);
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto compute = [&](const Stage& st, int b) {
    wave_sync();  // the previous superblock's scale reads are done
    lds_ds[lane] = QmfDs{(double)h2f(st.ds & 0xFFFFu), (double)h2f(st.ds >> 16)};
    wave_sync();
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const qmf_v4i a = qmf_v4i{(int)(st.a[g].x & amask), (int)(st.a[g].y & amask),
                                (int)(st.a[g].z & amask), (int)(st.a[g].w & amask)};
      const qmf_v4i z4 = {0, 0, 0, 0};
      qmf_v16i C = {0};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        qmf_v4i bq;
        if constexpr (T == Q4_K) {
          // sub-block 4g + jj: quarter 2g + jj/2, low (jj even) or high nibbles
          const u32x4 v = st.q[2 * g + (jj >> 1)];
          const int sh = 4 * (jj & 1);
          bq = qmf_v4i{(int)((v.x >> sh) & 0x0F0F0F0Fu), (int)((v.y >> sh) & 0x0F0F0F0Fu),
                       (int)((v.z >> sh) & 0x0F0F0F0Fu), (int)((v.w >> sh) & 0x0F0F0F0Fu)};
        } else {
          // sub-block 4g + jj: this lane's K-slice is the low (s = 0) or high
          // nibbles of its 16 bytes, looked up in the codebook
          const u32x4 v = st.q[4 * g + jj];
          const int sh = 4 * s;
          bq = qmf_v4i{(int)iq4nl_lookup(v.x >> sh), (int)iq4nl_lookup(v.y >> sh),
                       (int)iq4nl_lookup(v.z >> sh), (int)iq4nl_lookup(v.w >> sh)};
        }
        C = __builtin_amdgcn_mfma_i32_32x32x32_i8(slot == jj ? a : z4, bq, C, 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = 4 * g + jj;
        // scale (and Q4_K min) of sub-block j, as qmv_tile's decode_sub computes them
        double wsc, wmn = 0.0;
        if constexpr (T == Q4_K) q4k_scales(st.h, j, wsc, wmn);
        else wsc = iq4xs_scale(st.h.x, st.h.y, j);
        // rows m >= M (upper-half lanes at M = 7) drain zero dots against
        // row 0's scales and are never stored
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const int m = 4 * s + mm;
          const QmfDs e = lds_ds[(m < M ? m : 0) * 8 + j];
          const int I = C[4 * jj + mm];
          acc[j >> 1][mm] = fma(wsc * e.d, (double)I, acc[j >> 1][mm]);
          if constexpr (T == Q4_K) acc[j >> 1][mm] = fma(wmn, e.s, acc[j >> 1][mm]);
          if (DUMP && m < M && nrow < N)
            isums[((size_t)m * N + nrow) * (K / SUB) + (size_t)b * (QK / SUB) + j] = I;
        }
      }
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(S[d], wave + d * P);
  const int niter = (((nsb + P - 1) / P) + DEPTH - 1) / DEPTH * DEPTH;
  auto step = [&](Stage& st, int ii, bool refill) {
    const int b = wave + ii * P;
    if (b < nsb) compute(st, b);
    if (refill) fetch(st, b + DEPTH * P);
  };
  int i = 0;
  for (; i + DEPTH < niter; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, true);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) step(S[d], i + d, false);

  // quarters in qmv_tile's order ((q0 + q1) + (q2 + q3)), then the waves in order
  double* red = reinterpret_cast<double*>(smem);
  __syncthreads();  // the staging area is reused for the reduction
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int m = 4 * s + mm;
    if (m < M) red[(wave * QMF_ROWS + n) * M + m] = (acc[0][mm] + acc[1][mm]) + (acc[2][mm] + acc[3][mm]);
  }
  __syncthreads();
  for (int o = tid; o < QMF_ROWS * M; o += 64 * P) {
    const int m = o % M, r = o / M;
    double v = red[r * M + m];
    for (int w = 1; w < P; ++w) v += red[(w * QMF_ROWS + r) * M + m];
    if (n0 + r < N) y[(size_t)m * N + n0 + r] = (float)v;
  }
}

// ------------------------------------- the MFMA tile for M = 9..16
//
// qmf_tile's sums for up to 16 activation rows (Q4_K and IQ4_XS through
// qdot_qmatmul): the A tile holds two slots of 16 rows, the MFMA of
// sub-block 2q + jj fills slot jj, so one group of two MFMAs is one quarter,
// and result register r of lane l holds activation row (8(r/4)) % 16 + 4s +
// r%4 of sub-block 2q + (8(r/4))/16.  Each lane drains its eight rows into
// per-quarter fp64 chains in qmf_tile's (and qmv_tile's) order, so rows are
// bitwise the same for every M = 1..16.
template <int T, int M, int DEPTH, bool DUMP>
__device__ __forceinline__ void qmf16_tile(const uint8_t* __restrict__ W, int N, int K,
                                         const uint8_t* __restrict__ xq, float* __restrict__ y,
                                         int32_t* __restrict__ isums, int tile, uint8_t* smem) {
  static_assert(qmf_type<T>(), "the MFMA decode tile takes Q4_K or IQ4_XS weights");
  static_assert(M <= QMF_MAX_M, "the MFMA decode tile holds at most 16 activation rows");
  // A-tile geometry: R activation rows per slot, S = 32/R slots, so one group
  // of S MFMAs covers S consecutive sub-blocks.  With R = 16 (M = 9..16) a
  // group is two sub-blocks, one quarter; the same code with R = 8 is
  // qmf_tile's geometry.
  constexpr int R = qmf_rows<M>();
  constexpr int S = 32 / R;
  constexpr int G = 8 / S;          // groups per superblock
  constexpr int MM = R / 2;         // activation rows per lane (two sets of four)
  constexpr int NDS = 8 * R / 64;   // scale entries each lane publishes per superblock
  constexpr int NQ = T == Q4_K ? 4 : 8;  // 16-byte code loads per superblock and lane
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int SUB = Geom<T>::SUB;
  const int P = blockDim.x >> 6;
  const int nsb = K / QK;
  const int nq8 = K / Q8_BLOCK;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, s = lane >> 5;
  const int slot = (lane & 31) / R, mrow = (lane & 31) % R;  // this lane's A row: block slot, activation row
  const int n0 = tile * QMF_ROWS;
  const int nrow = n0 + n;
  const uint8_t* wrow = W + (size_t)(nrow < N ? nrow : N - 1) * nsb * BYTES;
  // this lane's A data: row mrow.  Rows >= M read row 0 (A data and scales),
  // so they compute row 0's finite sums, which are never stored: the loop
  // below is the same code for every M.
  const uint8_t* xa_row = xq + ((size_t)(mrow < M ? mrow : 0) * nq8 + slot) * Q8_BYTES + 4 + 16 * s;
  // scale entries this lane publishes per superblock: e = lane + 64u holds
  // activation row e/8, block e%8
  const uint8_t* xd_src[NDS];
#pragma unroll
  for (int u = 0; u < NDS; ++u) {
    const int e = lane + 64 * u, dm = e >> 3, dj = e & 7;
    xd_src[u] = xq + ((size_t)(dm < M ? dm : 0) * nq8 + dj) * Q8_BYTES;
  }
  QmfDs* lds_ds = reinterpret_cast<QmfDs*>(smem) + wave * 8 * R;

  double acc[4][MM];  // [quarter][activation row of this lane]
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) acc[q][mm] = 0.0;

  // Q4_K: header (d, dmin, scales) and the code bytes of K-slice s of each
  // quarter (low nibbles sub-block 2q, high 2q+1).  IQ4_XS: header (d,
  // scales_h, scales_l) and the 16 code bytes of each sub-block (low nibbles
  // its elements 0-15 = K-slice 0, high nibbles 16-31 = K-slice 1).
  struct Stage {
    u32x4 h, q[NQ];
    u32x4 a[G];       // this lane's A data in each group
    uint32_t ds[NDS]; // d, s of the published scale entries
  };
  Stage St[DEPTH];
  auto fetch = [&](Stage& st, int bsb) {
    const int bc = bsb < nsb ? bsb : nsb - 1;
    const uint8_t* sb = wrow + (size_t)bc * BYTES;
    st.h = ld16(sb);
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      st.q[q] = T == Q4_K ? ld16(sb + 16 + 32 * q + 16 * s) : ld16(sb + 8 + 16 * q);
#pragma unroll
    for (int g = 0; g < G; ++g) st.a[g] = ld16(xa_row + (size_t)(8 * bc + S * g) * Q8_BYTES);
#pragma unroll
    for (int u = 0; u < NDS; ++u) st.ds[u] = ld4(xd_src[u] + (size_t)8 * bc * Q8_BYTES);
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto compute = [&](const Stage& st, int b) {
    wave_sync();  // the previous superblock's scale reads are done
#pragma unroll
    for (int u = 0; u < NDS; ++u)
      lds_ds[lane + 64 * u] = QmfDs{(double)h2f(st.ds[u] & 0xFFFFu), (double)h2f(st.ds[u] >> 16)};
    wave_sync();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const qmf_v4i a = qmf_v4i{(int)st.a[g].x, (int)st.a[g].y, (int)st.a[g].z, (int)st.a[g].w};
      const qmf_v4i z4 = {0, 0, 0, 0};
      qmf_v16i C = {0};
#pragma unroll
      for (int jj = 0; jj < S; ++jj) {
        const int j = S * g + jj;  // sub-block
        qmf_v4i bq;
        if constexpr (T == Q4_K) {
          // sub-block j: quarter j/2, low (j even) or high nibbles
          const u32x4 v = st.q[j >> 1];
          const int sh = 4 * (j & 1);
          bq = qmf_v4i{(int)((v.x >> sh) & 0x0F0F0F0Fu), (int)((v.y >> sh) & 0x0F0F0F0Fu),
                       (int)((v.z >> sh) & 0x0F0F0F0Fu), (int)((v.w >> sh) & 0x0F0F0F0Fu)};
        } else {
          // sub-block j: this lane's K-slice is the low (s = 0) or high
          // nibbles of its 16 bytes, looked up in the codebook
          const u32x4 v = st.q[j];
          const int sh = 4 * s;
          bq = qmf_v4i{(int)iq4nl_lookup(v.x >> sh), (int)iq4nl_lookup(v.y >> sh),
                       (int)iq4nl_lookup(v.z >> sh), (int)iq4nl_lookup(v.w >> sh)};
        }
        C = __builtin_amdgcn_mfma_i32_32x32x32_i8(slot == jj ? a : z4, bq, C, 0, 0, 0);
      }
#pragma unroll
      for (int jj = 0; jj < S; ++jj) {
        const int j = S * g + jj;
        // scale (and Q4_K min) of sub-block j, as qmv_tile's decode_sub computes them
        double wsc, wmn = 0.0;
        if constexpr (T == Q4_K) q4k_scales(st.h, j, wsc, wmn);
        else wsc = iq4xs_scale(st.h.x, st.h.y, j);
        // Result register r of lane l holds A row 8(r/4) + 4s + r%4, i.e.
        // slot (8(r/4))/R -- the registers of slot jj carry sub-block j --
        // and activation row m = (8(r/4)) % R + 4s + r%4.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if ((8 * (r >> 2)) / R != jj) continue;
          const int mm = (((8 * (r >> 2)) % R) >> 1) + (r & 3);   // 0..MM-1
          const int m = (8 * (r >> 2)) % R + 4 * s + (r & 3);
          const QmfDs e = lds_ds[m * 8 + j];
          const int I = C[r];
          acc[j >> 1][mm] = fma(wsc * e.d, (double)I, acc[j >> 1][mm]);
          if constexpr (T == Q4_K) acc[j >> 1][mm] = fma(wmn, e.s, acc[j >> 1][mm]);
          if (DUMP && m < M && nrow < N)
            isums[((size_t)m * N + nrow) * (K / SUB) + (size_t)b * (QK / SUB) + j] = I;
        }
      }
    }
  };

#pragma unroll
  for (int d = 0; d < DEPTH; ++d) fetch(St[d], wave + d * P);
  const int niter = (((nsb + P - 1) / P) + DEPTH - 1) / DEPTH * DEPTH;
  auto step = [&](Stage& st, int ii, bool refill) {
    const int b = wave + ii * P;
    if (b < nsb) compute(st, b);
    if (refill) fetch(st, b + DEPTH * P);
  };
  int i = 0;
  for (; i + DEPTH < niter; i += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) step(St[d], i + d, true);
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) step(St[d], i + d, false);

  // quarters in qmv_tile's order ((q0 + q1) + (q2 + q3)), then the waves in order
  double* red = reinterpret_cast<double*>(smem);
  __syncthreads();  // the staging area is reused for the reduction
#pragma unroll
  for (int mm = 0; mm < MM; ++mm) {
    const int m = 8 * (mm >> 2) + 4 * s + (mm & 3);
    if (m < M) red[(wave * QMF_ROWS + n) * M + m] = (acc[0][mm] + acc[1][mm]) + (acc[2][mm] + acc[3][mm]);
  }
  __syncthreads();
  for (int o = tid; o < QMF_ROWS * M; o += 64 * P) {
    const int m = o % M, r = o / M;
    double v = red[r * M + m];
    for (int w = 1; w < P; ++w) v += red[(w * QMF_ROWS + r) * M + m];
    if (n0 + r < N) y[(size_t)m * N + n0 + r] = (float)v;
  }
}

// LDS bytes of a workgroup of `waves` waves running the MFMA tile (mfma) or
// the dot4 tile.
template <int M> inline size_t qmv_lds_bytes_tile(bool mfma, int waves) {
  const size_t stage = (size_t)waves * (mfma ? (size_t)8 * qmf_rows<M>() * sizeof(QmfDs)
                                             : (size_t)8 * M * (Q8_BLOCK + sizeof(DsEntry)));
  const size_t red = (size_t)waves * (mfma ? QMF_ROWS : QMV_SLOTS) * M * sizeof(double);
  return stage > red ? stage : red;
}
template <int T, int M> inline size_t qmv_lds_bytes(int waves) {
  return qmv_lds_bytes_tile<M>(qmf_ok<T, M>(), waves);
}

template <int T, int M, int DEPTH, bool DUMP, bool XF = false>
__global__ __launch_bounds__(QMV_MAX_THREADS) void qmv_kernel(
    const uint8_t* __restrict__ W, int N, int K, const uint8_t* __restrict__ xq,
    float* __restrict__ y, int32_t* __restrict__ isums) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  if constexpr (XF)
    qmv_tile<T, M, DEPTH, false, true>(W, N, K, xq, y, nullptr, blockIdx.x, smem);
  else if constexpr (M > 8)
    qmf16_tile<T, M, DEPTH, DUMP>(W, N, K, xq, y, isums, blockIdx.x, smem);
  else if constexpr (qmf_ok<T, M>())
    qmf_tile<T, M, DEPTH, DUMP>(W, N, K, xq, y, isums, blockIdx.x, smem);
  else if constexpr (q6f_ok<T, M>())
    q6f_tile<M, DEPTH, DUMP>(W, N, K, xq, y, isums, blockIdx.x, smem);
  else
    qmv_tile<T, M, DEPTH, DUMP>(W, N, K, xq, y, isums, blockIdx.x, smem);
}

// Several matrices that share the activation (same K and M) in one launch:
// workgroup g works on matrix i for tile_end[i-1] <= g < tile_end[i], with
// the same per-tile code, K split and summation order as a launch of that
// matrix alone, so every output is bitwise the one qmv_kernel gives.  Types
// TA and TB (equal for a single-type group) are the only ones present.
constexpr int QMV_MULTI_MAX = 4;
struct QmvMulti {
  const uint8_t* W[QMV_MULTI_MAX];
  float* y[QMV_MULTI_MAX];
  int N[QMV_MULTI_MAX];
  int type[QMV_MULTI_MAX];
  int tile_end[QMV_MULTI_MAX];
  int n;
};

// XF: fp32 activations quantized in the kernel (qmv_tile's XF mode; dot4
// tiles only).
template <int TA, int TB, int M, int DEPTH, bool MF, bool XF = false>
__global__ __launch_bounds__(QMV_MAX_THREADS) void qmv_multi_kernel(QmvMulti a, int K,
                                                                    const uint8_t* __restrict__ xq) {
  static_assert(!(XF && MF), "in-kernel quantization runs on the dot4 tile");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int g = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int j = 0; j < QMV_MULTI_MAX - 1; ++j)
    if (j < a.n - 1 && g >= a.tile_end[j]) i = j + 1;
  const int tile = g - (i > 0 ? a.tile_end[i - 1] : 0);
  if (TA == TB || a.type[i] == TA) {
    if constexpr (qmf_group_ok<TA, M, MF>())
      qmf_tile<TA, M, DEPTH, false>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
    else if constexpr (!XF && q6f_ok<TA, M>())
      q6f_tile<M, DEPTH, false>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
    else
      qmv_tile<TA, M, DEPTH, false, XF>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
  } else {
    if constexpr (qmf_group_ok<TB, M, MF>())
      qmf_tile<TB, M, DEPTH, false>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
    else if constexpr (!XF && q6f_ok<TB, M>())
      q6f_tile<M, DEPTH, false>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
    else
      qmv_tile<TB, M, DEPTH, false, XF>(a.W[i], a.N[i], K, xq, a.y[i], nullptr, tile, smem);
  }
}

// ------------------------------------------------ launch-shape helpers
// Waves per workgroup: a function of K only (the K split fixes the fp64
// summation order, which must not depend on M): about four superblocks per
// wave, rounded up to a power of two, at most eight waves.  (Measured on
// MI355X with K = 5120, 20 superblocks: eight waves beat five by 8-30 %.)
inline int qmv_waves(int nsb) {
  const int p = (nsb + 3) / 4;
  int q = 1;
  while (q < p && q < 8) q *= 2;
  return q;
}

// Superblocks in flight per wave (prefetch depth; it changes no arithmetic).
// Chosen by measurement on MI355X (Qwen3-8B shapes, M = 1..8): the weight
// bytes one stage of all waves puts in flight decide it.  About 7 MB per
// stage (12288 x 4096 Q4_K, 4096 x 12288 Q6_K) already saturates HBM with one
// stage at M <= 4; the 9 MB matrices want all four superblocks of a wave in
// flight; Q6_K's larger register stage is kept to two.
// Weight rows per workgroup of the decode kernels for (type, M).
inline int qmv_rows(int type, bool mfma) { return (mfma && (type == Q4_K || type == IQ4_XS)) ? QMF_ROWS : QMV_SLOTS; }

inline long qmv_stage_bytes(int type, int N, int K) {
  const long waves = (long)((N + QMV_SLOTS - 1) / QMV_SLOTS) * qmv_waves(K / QK);
  const int bytes = type == Q6_K ? 210 : (type == IQ4_XS ? 136 : (type == Q8_0 ? 272 : 144));
  return waves * QMV_SLOTS * (long)bytes;
}
inline int qmv_depth_for(long stage_bytes, int M, bool wide_stage) {
  int d;
  if (stage_bytes >= (4L << 20)) d = M <= 4 ? 1 : 2;
  else if (stage_bytes >= (3L << 20)) d = 2;
  else d = 4;
  if (wide_stage && d > 2) d = 2;
  return d;
}
// Prefetch depth of a launch with MFMA tiles (the stage holds a whole
// superblock per lane): one for the 28 MB-class matrices and groups (at
// least 4 MB in flight per stage), else two.  Measured on MI355X at M = 8:
// gate+up 18.6 us at depth 1 against 19.9 at 2; q+k+v 9.7 us at 2 against
// 10.7 at 1; depth 4 spills registers at M = 7.
inline int qmf_depth(long stage_bytes) { return stage_bytes >= (4L << 20) ? 1 : 2; }

inline int qmv_depth(int type, int M, int N, int K) {
  return qmv_depth_for(qmv_stage_bytes(type, N, K), M, type == Q6_K || type == Q8_0);
}

}  // namespace qdot
