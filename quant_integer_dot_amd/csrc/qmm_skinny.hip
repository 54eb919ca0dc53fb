// qmm_skinny.hip -- mid-batch matmul (9 <= M <= 96 activation rows) on the
// int8 matrix cores: v_mfma_i32_16x16x32_i8, sixteen activation rows per tile.
//
// Same arithmetic as the other kernels: exact int32 block dots of the raw
// weight codes with the Q8_1 activations, then exact-term fp64 scale drains
// (Kestrel section 5: exact int32 inside the block, scales after).  What
// differs is the shape of the work.  At mid-batch M the weights must still be
// read from HBM once (the V100TPS log measured the per-token matvec falling
// behind a batched kernel from M ~ 15, 2026-08-12 entries), but an M = 512
// style tile of 128 activation rows wastes most of its drain work on padding,
// and one 32 x 64 tile per wave over all of K leaves too few, too long waves.
// Here a wave owns 16 activation rows x 16 or 32 weight rows (one or two
// 16 x 16 tiles) and a workgroup of eight waves splits K eight ways, so each
// wave drains only two superblocks of K = 4096 and the grid covers the chip.
//
// Lane layout of v_mfma_i32_16x16x32_i8 (measured on gfx950): operand lane l
// supplies row (A) / column (B) l%16 and K-slice l/16 (8 bytes); result
// register r of lane l holds D[4*(l/16) + r][l%16].  A = activation codes
// (rows m), B = weight codes (columns n), so each lane drains 4 activation
// rows x 1 weight row per tile: the weight scales of a lane's column come
// from one LDS read per tile and block, the activation scales of its 4 rows
// from four.  Both scale tables are fp64 and rebuilt per superblock.
#include <type_traits>

#include "formats.hpp"

namespace qdot {

typedef int v4i_s __attribute__((ext_vector_type(4)));

constexpr int SK_WAVES = 8;   // waves per workgroup = K slices
constexpr int SK_BM = 16;     // activation rows per workgroup
constexpr int SK_XCDS = 8;

// LDS entry of the weight-scale table: Q4_K (d*sc, -dmin*m); IQ4_XS, Q4_0,
// Q8_0 (scale, 0); Q6_K (d, and the two int8 sub-scales of the block).
struct __attribute__((aligned(16))) SkW {
  double w;
  union {
    double mn;
    int s01[2];
  };
};
struct __attribute__((aligned(16))) SkA { double d, s; };  // activation D, S

__device__ __forceinline__ long sk_pack(uint32_t lo, uint32_t hi) {
  return (long)((uint64_t)lo | ((uint64_t)hi << 32));
}
__device__ __forceinline__ uint32_t sk_ld2(const uint8_t* p) {
  unsigned short v;
  __builtin_memcpy(&v, p, 2);
  return v;
}

// ----------------------------------------------------------- per format
// Raw: what lane (c16, s) loads per superblock for one weight row -- the
// K-slice s bytes of all eight blocks and the fields its scale entries need
// (entries for blocks 2s and 2s+1).  codes(raw, j, s): the 8 signed int8
// codes of K-slice s of block j.  entry(raw, u): the weight-scale entry of
// block 2s+u.
template <int T> struct Sk;

template <> struct Sk<Q4_K> {
  struct Raw { u32x2 q[4]; u32x4 h; };  // qs pair c, K-slice s; header
  __device__ static Raw load(const uint8_t* sb, int s) {
    Raw r;
#pragma unroll
    for (int c = 0; c < 4; ++c) r.q[c] = ld8(sb + 16 + 32 * c + 8 * s);
    r.h = ld16(sb);
    return r;
  }
  template <int J> __device__ static long codes(const Raw& r, int) {
    const u32x2 v = r.q[J >> 1];
    constexpr int sh = (J & 1) ? 4 : 0;
    return sk_pack((v.x >> sh) & 0x0F0F0F0Fu, (v.y >> sh) & 0x0F0F0F0Fu);
  }
  __device__ static SkW entry(const Raw& r, int j) {
    SkW e;
    q4k_scales(r.h, j, e.w, e.mn);  // d*sc, -dmin*m
    return e;
  }
};

template <> struct Sk<IQ4_XS> {
  struct Raw { u32x2 q[8]; u32x2 h; };
  __device__ static Raw load(const uint8_t* sb, int s) {
    Raw r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.q[j] = ld8(sb + 8 + 16 * j + 8 * (s & 1));
    r.h = ld8(sb);
    return r;
  }
  template <int J> __device__ static long codes(const Raw& r, int s) {
    const int sh = (s >> 1) ? 4 : 0;
    return sk_pack(iq4nl_lookup(r.q[J].x >> sh), iq4nl_lookup(r.q[J].y >> sh));
  }
  __device__ static SkW entry(const Raw& r, int j) {
    SkW e;
    e.w = iq4xs_scale(r.h.x, r.h.y, j);
    e.mn = 0.0;
    return e;
  }
};

template <> struct Sk<Q4_0> {
  struct Raw { u32x2 q[8]; uint32_t d[2]; };
  __device__ static Raw load(const uint8_t* sb, int s) {
    Raw r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.q[j] = ld8(sb + 18 * j + 2 + 8 * (s & 1));
    r.d[0] = sk_ld2(sb + 18 * (2 * s));
    r.d[1] = sk_ld2(sb + 18 * (2 * s + 1));
    return r;
  }
  template <int J> __device__ static long codes(const Raw& r, int s) {
    const int sh = (s >> 1) ? 4 : 0;
    return sk_pack(q40_signed((r.q[J].x >> sh) & 0x0F0F0F0Fu), q40_signed((r.q[J].y >> sh) & 0x0F0F0F0Fu));
  }
  __device__ static SkW entry(const Raw& r, int j) {
    SkW e;
    e.w = (double)h2f(r.d[j & 1]);
    e.mn = 0.0;
    return e;
  }
};

template <> struct Sk<Q8_0> {
  struct Raw { u32x2 q[8]; uint32_t d[2]; };
  __device__ static Raw load(const uint8_t* sb, int s) {
    Raw r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.q[j] = ld8(sb + 34 * j + 2 + 8 * s);
    r.d[0] = sk_ld2(sb + 34 * (2 * s));
    r.d[1] = sk_ld2(sb + 34 * (2 * s + 1));
    return r;
  }
  template <int J> __device__ static long codes(const Raw& r, int) {
    return sk_pack(r.q[J].x, r.q[J].y);
  }
  __device__ static SkW entry(const Raw& r, int j) {
    SkW e;
    e.w = (double)h2f(r.d[j & 1]);
    e.mn = 0.0;
    return e;
  }
};

template <> struct Sk<Q6_K> {
  // element e = 32j + 8s + i: h = j/4, g = j%4; low 4 bits from
  // ql[64h + 32(g&1) + 8s + i] (>> 4 if g >= 2), high 2 bits from
  // qh[32h + 8s + i] >> 2g; code - 32.  Blocks g and g+2 share their ql
  // bytes and all four g of one h share the qh bytes.
  struct Raw { u32x2 l[4]; u32x2 q[2]; uint32_t sc; uint32_t d; };
  __device__ static Raw load(const uint8_t* sb, int s) {
    Raw r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r.l[2 * h] = ld8(sb + 64 * h + 8 * s);
      r.l[2 * h + 1] = ld8(sb + 64 * h + 32 + 8 * s);
      r.q[h] = ld8(sb + 128 + 32 * h + 8 * s);
    }
    r.sc = ld4(sb + 192 + 4 * s);  // int8 sub-scales of blocks 2s, 2s+1
    r.d = sk_ld2(sb + 208);
    return r;
  }
  template <int J> __device__ static long codes(const Raw& r, int) {
    constexpr int h = J >> 2, g = J & 3;
    const u32x2 l = r.l[2 * h + (g & 1)];
    const u32x2 q = r.q[h];
    return sk_pack(q6k_signed(q6k_code<(g >= 2)>(l.x, q.x, g & 1)),
                   q6k_signed(q6k_code<(g >= 2)>(l.y, q.y, g & 1)));
  }
  __device__ static SkW entry(const Raw& r, int j) {
    const uint32_t sc = r.sc >> (16 * (j & 1));
    SkW e;
    e.w = (double)h2f(r.d);
    e.s01[0] = (int)(int8_t)(sc & 0xFFu);
    e.s01[1] = (int)(int8_t)((sc >> 8) & 0xFFu);
    return e;
  }
};

// ------------------------------------------------------------------ kernel
template <int T, int SK_NT, bool DUMP>
__global__ __launch_bounds__(64 * SK_WAVES) void qmm_skinny_kernel(
    const uint8_t* __restrict__ W, int N, int K, const uint8_t* __restrict__ xq, int M,
    float* __restrict__ y, int32_t* __restrict__ isums, int m_tiles, int n_groups) {
  using F = Sk<T>;
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int SUB = Geom<T>::SUB;
  constexpr int SK_BN = 16 * SK_NT;  // weight rows per workgroup
  // Per wave: weight-scale table [tile][block][row16] and activation-scale
  // table [block][row16]; after the main loop the same memory holds the
  // K-slice partial sums for the reduction.
  constexpr int WTAB = SK_NT * 8 * 16;
  constexpr int ATAB = 8 * 16;
  constexpr int TAB_BYTES = (WTAB * sizeof(SkW) + ATAB * sizeof(SkA)) * SK_WAVES;
  constexpr int RED_BYTES = (SK_WAVES - 1) * SK_NT * 4 * 64 * 8;
  __shared__ __align__(16) uint8_t lds[TAB_BYTES > RED_BYTES ? TAB_BYTES : RED_BYTES];

  // XCD-aware order: the m-tiles of one weight tile share the residue mod 8.
  const int id = blockIdx.x;
  const int xcd = id % SK_XCDS, local = id / SK_XCDS;
  const int m_tile = local % m_tiles;
  const int n_group = (local / m_tiles) * SK_XCDS + xcd;
  if (n_group >= n_groups) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c16 = lane & 15, s = lane >> 4;  // operand row/column, K-slice
  const int nsb = K / QK, nq8 = K / Q8_BLOCK;
  const size_t row_bytes = (size_t)nsb * BYTES;
  const int m0 = m_tile * SK_BM;
  const int n0 = n_group * SK_BN;

  SkW* wtab = reinterpret_cast<SkW*>(lds) + (size_t)wave * WTAB;
  SkA* atab = reinterpret_cast<SkA*>(lds + (size_t)SK_WAVES * WTAB * sizeof(SkW)) + (size_t)wave * ATAB;

  // this lane's activation row (A operand) and weight rows (B operand, one per
  // tile); rows past the edges are clamped and never stored
  const int ma = m0 + c16 < M ? m0 + c16 : M - 1;
  const uint8_t* xrow = xq + (size_t)ma * nq8 * Q8_BYTES;
  const uint8_t* wrow[SK_NT];
#pragma unroll
  for (int t = 0; t < SK_NT; ++t) {
    const int n = n0 + 16 * t + c16;
    wrow[t] = W + (size_t)(n < N ? n : N - 1) * row_bytes;
  }

  // Everything one superblock needs, loaded as one stage: the weight bytes
  // and scale fields of four rows, the activation K-slices of eight blocks
  // and the scales of the lane's two blocks.
  struct Stage {
    typename F::Raw w[SK_NT];
    u32x2 a[8];
    uint32_t ds[2];
  };
  auto fetch = [&](Stage& st, int bsb) {
    const int bc = bsb < nsb ? bsb : nsb - 1;  // clamped: a last redundant fetch stays in bounds
#pragma unroll
    for (int t = 0; t < SK_NT; ++t) st.w[t] = F::load(wrow[t] + (size_t)bc * BYTES, s);
    const uint8_t* xb = xrow + (size_t)bc * 8 * Q8_BYTES;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.a[j] = ld8(xb + j * Q8_BYTES + 4 + 8 * s);
    st.ds[0] = ld4(xb + (2 * s) * Q8_BYTES);
    st.ds[1] = ld4(xb + (2 * s + 1) * Q8_BYTES);
  };

  double acc[SK_NT][4];
#pragma unroll
  for (int t = 0; t < SK_NT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] = 0.0;

  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  auto compute = [&](const Stage& st, int b) {
    // ---- scale tables of this superblock: lane (c16, s) fills blocks 2s, 2s+1
    wave_sync();  // the previous superblock's table reads are done
#pragma unroll
    for (int t = 0; t < SK_NT; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) wtab[(t * 8 + 2 * s + u) * 16 + c16] = F::entry(st.w[t], 2 * s + u);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      atab[(2 * s + u) * 16 + c16] = SkA{(double)h2f(st.ds[u] & 0xFFFFu), (double)h2f(st.ds[u] >> 16)};
    wave_sync();

    auto do_block = [&](auto JC) {
      constexpr int j = decltype(JC)::value;
      const long a = sk_pack(st.a[j].x, st.a[j].y);
      SkA ae[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ae[r] = atab[j * 16 + 4 * s + r];
#pragma unroll
      for (int t = 0; t < SK_NT; ++t) {
        const long bw = F::template codes<j>(st.w[t], s);
        const SkW we = wtab[(t * 8 + j) * 16 + c16];
        const v4i_s z = {0, 0, 0, 0};
        if constexpr (T == Q6_K) {
          // two 16-element sub-blocks: one MFMA each, the other half of the
          // activation K-slices zeroed
          const long a0 = s < 2 ? a : 0L, a1 = s < 2 ? 0L : a;
          const v4i_s I0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, bw, z, 0, 0, 0);
          const v4i_s I1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(a1, bw, z, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int P = q6k_pair(we.s01[0], I0[r], we.s01[1], I1[r]);  // exact int
            acc[t][r] = fma(we.w * ae[r].d, (double)P, acc[t][r]);
            if (DUMP) {
              const int m = m0 + 4 * s + r, n = n0 + 16 * t + c16;
              if (m < M && n < N) {
                int32_t* p = isums + ((size_t)m * N + n) * (K / SUB) + (size_t)b * (QK / SUB) + 2 * j;
                p[0] = I0[r];
                p[1] = I1[r];
              }
            }
          }
        } else {
          const v4i_s I = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, bw, z, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            acc[t][r] = fma(we.w * ae[r].d, (double)I[r], acc[t][r]);  // exact product
            if constexpr (T == Q4_K) acc[t][r] = fma(we.mn, ae[r].s, acc[t][r]);
            if (DUMP) {
              const int m = m0 + 4 * s + r, n = n0 + 16 * t + c16;
              if (m < M && n < N)
                isums[((size_t)m * N + n) * (K / SUB) + (size_t)b * (QK / SUB) + j] = I[r];
            }
          }
        }
      }
    };
    do_block(std::integral_constant<int, 0>{});
    do_block(std::integral_constant<int, 1>{});
    do_block(std::integral_constant<int, 2>{});
    do_block(std::integral_constant<int, 3>{});
    do_block(std::integral_constant<int, 4>{});
    do_block(std::integral_constant<int, 5>{});
    do_block(std::integral_constant<int, 6>{});
    do_block(std::integral_constant<int, 7>{});
  };

  // One stage: all of a superblock's loads are issued together, before its
  // scale tables are built (two stages in flight spill registers).
  for (int b = wave; b < nsb; b += SK_WAVES) {
    Stage st;
    fetch(st, b);
    compute(st, b);
  }

  // ---- K-slice partials through LDS, added in slice order by wave 0
  __syncthreads();  // every wave is done with its tables
  double* red = reinterpret_cast<double*>(lds);
  auto slot = [&](int k, int t, int r) { return (((k - 1) * SK_NT + t) * 4 + r) * 64 + lane; };
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < SK_NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[slot(wave, t, r)] = acc[t][r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll 1
  for (int k = 1; k < SK_WAVES; ++k)
#pragma unroll
    for (int t = 0; t < SK_NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] += red[slot(k, t, r)];
#pragma unroll
  for (int t = 0; t < SK_NT; ++t) {
    const int n = n0 + 16 * t + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 4 * s + r;
      if (m < M && n < N) y[(size_t)m * N + n] = (float)acc[t][r];
    }
  }
}

template <int T, int NT, bool DUMP>
static int launch_skinny_t(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                           int32_t* isums, hipStream_t s) {
  const int m_tiles = (M + SK_BM - 1) / SK_BM;
  const int n_groups = (N + 16 * NT - 1) / (16 * NT);
  const long groups = (long)(n_groups + SK_XCDS - 1) / SK_XCDS;
  const long grid = (long)SK_XCDS * m_tiles * groups;
  if (grid > 0x7FFFFFFFL) return -1;
  hipLaunchKernelGGL((qmm_skinny_kernel<T, NT, DUMP>), dim3((unsigned)grid), dim3(64 * SK_WAVES), 0, s,
                     W, N, K, xq, M, y, isums, m_tiles, n_groups);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Weight tiles per wave: two where that still leaves at least 144 workgroups,
// else one.  Measured on MI355X at M = 9..64: 4096 x 4096 and 4096 x 12288
// at M = 16 (128 workgroups of two tiles) run 1.4-1.6x slower with two tiles;
// 7168 x 5120 and 5120 x 17408 at M = 16 (224 and 160) run 1.1-1.2x faster
// with two, as does every shape with 256 or more.  The choice changes no
// summation order.
template <int T, bool DUMP>
static int launch_skinny_n(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                           int32_t* isums, hipStream_t s) {
  const long m_tiles = (M + SK_BM - 1) / SK_BM;
  const bool two = m_tiles * ((N + 31) / 32) >= 144;
  if (two) return launch_skinny_t<T, 2, DUMP>(W, N, K, xq, M, y, isums, s);
  return launch_skinny_t<T, 1, DUMP>(W, N, K, xq, M, y, isums, s);
}

int launch_qmm_skinny(const void* W, int type, int N, int K, const void* xq, int M, float* y,
                      int32_t* isums, hipStream_t s) {
  const uint8_t* w8 = static_cast<const uint8_t*>(W);
  const uint8_t* x8 = static_cast<const uint8_t*>(xq);
  const bool dump = isums != nullptr;
  switch (type) {
#define SK_CASE(TT)                                                              \
  case TT:                                                                       \
    return dump ? launch_skinny_n<TT, true>(w8, N, K, x8, M, y, isums, s)        \
                : launch_skinny_n<TT, false>(w8, N, K, x8, M, y, isums, s);
    SK_CASE(Q4_K)
    SK_CASE(Q6_K)
    SK_CASE(IQ4_XS)
    SK_CASE(Q4_0)
    SK_CASE(Q8_0)
#undef SK_CASE
    default:
      return -2;
  }
}

}  // namespace qdot
