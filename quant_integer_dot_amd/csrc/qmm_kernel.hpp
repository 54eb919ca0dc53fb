// qmm_kernel.hpp -- prefill matmul for M > 8 activation rows (row a6 of the hot
// path), on the int8 matrix cores of gfx950.
//
// Same arithmetic as the decode kernel -- exact int32 block dots of the raw
// weight codes with the Q8_1 activations, then exact-term fp64 scale drains
// (Kestrel section 5: exact int32 inside the block, scales after) -- but the
// block dots of a 32 x 32 output tile come from one MFMA per 32-element
// block: v_mfma_i32_32x32x32_i8 for IQ4_XS, Q4_0 and Q8_0 (one MFMA = one
// sub-block), two v_mfma_i32_32x32x16_i8 for Q6_K (16-element sub-blocks).
// Q4_K runs on 16 x 16 tiles with its min term on the fp64 matrix cores (its
// own tile, further down).
// The V100 pages found dequantize + dense GEMM faster than their dp4a kernel
// above M ~ 32-64 and their fused WMMA attempts slower than dp4a because the
// dequantized tile went through shared memory (V100TPS, "fp16 vs Q4
// crossover" and the fused-WMMA entry).  Here the int8 codes go straight from
// VGPRs into the MFMA and only the per-block scales are applied on the VALU.
//
// MFMA lane layout (measured on gfx950): operand lane l supplies row
// (A) / column (B) l%32 and K-slice l/32 (16 bytes for K=32, 8 for K=16); the
// bytes of A and B lanes pair by position.  Result register r of lane l holds
// D[8*(r/4) + 4*(l/32) + r%4][l%32].  A = activations (rows m), B = weight
// codes (columns n), so a lane's 16 outputs share one weight row and need 16
// activation scales, which the wave stages in LDS as fp64.
//
// Tiles: a workgroup has QMM_WAVES waves and covers 32*QMM_WAVES/KP
// activation rows by QMM_BN weight rows (QMM_NT MFMA tiles per wave).  Wave
// w takes the 32 rows (w / KP) and the superblocks b = w % KP (mod KP) of K;
// the KP partial sums of an output are added in fixed order at the end.  KP
// depends on N and K only, so an output's value does not depend on M.  The
// weight superblocks of each step are staged in LDS for the whole workgroup
// (coalesced copies, one copy for the waves that share a K slice); the
// activation codes go from HBM/L2 straight into VGPRs through a small ring.
#pragma once
#include <type_traits>

#include "formats.hpp"

namespace qdot {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int QMM_WAVES = 4;             // waves per workgroup
constexpr int QMM_NT = 2;                // 32-row weight tiles per wave
constexpr int QMM_BN = 32 * QMM_NT;      // weight rows per workgroup
constexpr int QMM_XCDS = 8;              // MI355X: 8 XCDs, workgroups dealt round-robin

struct QmmDs { double d, s; };  // one Q8_1 block's scales, fp64 (Q6_K uses d only)

// Result register r of lane l -> row of the 32 x 32 tile.
__device__ __forceinline__ int mfma_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// -------------------------------------------------------------- per format
// Per weight row and superblock: the scale fields.  Per weight row and
// 32-element block: the B operand data of this lane's K-slice g.
template <int T> struct QmmFmt;

template <> struct QmmFmt<IQ4_XS> {
  static constexpr int BYTES = 136;
  struct Hdr { u32x2 h; };
  struct Blk { u32x4 qs; };  // qs[16j .. 16j+16]: low nibbles elements 0-15, high 16-31
  __device__ static Hdr hdr(const uint8_t* sb) { return Hdr{ld8(sb)}; }
  __device__ static Blk blk(const uint8_t* sb, int j, int /*g*/) { return Blk{ld16(sb + 8 + 16 * j)}; }
  template <int J> __device__ static double scale(const Hdr& x, const Blk&) {
    return iq4xs_scale(x.h.x, x.h.y, J);
  }
  template <int J> __device__ static v4i codes(const Blk& b, int g) {
    const u32x4 v = b.qs;
    const int s = g ? 4 : 0;
    return v4i{(int)iq4nl_lookup(v.x >> s), (int)iq4nl_lookup(v.y >> s), (int)iq4nl_lookup(v.z >> s),
               (int)iq4nl_lookup(v.w >> s)};
  }
};

// Q4_0 / Q8_0: no superblock header; each 32-weight block carries its own
// fp16 d, loaded with the block's codes.
template <> struct QmmFmt<Q4_0> {
  static constexpr int BYTES = 8 * 18;
  struct Hdr {};
  struct Blk { u32x4 qs; uint32_t d; };  // qs[0..15] of block j; K-slice g = low / high nibbles
  __device__ static Hdr hdr(const uint8_t*) { return Hdr{}; }
  __device__ static Blk blk(const uint8_t* sb, int j, int /*g*/) {
    unsigned short dh;
    __builtin_memcpy(&dh, sb + 18 * j, 2);
    return Blk{ld16(sb + 18 * j + 2), dh};
  }
  template <int J> __device__ static double scale(const Hdr&, const Blk& b) { return (double)h2f(b.d); }
  // nibble q (0..15) -> int8 q - 8, four bytes at once without borrows
  template <int J> __device__ static v4i codes(const Blk& b, int g) {
    const int s = g ? 4 : 0;
    auto c = [&](uint32_t v) { return (int)q40_signed((v >> s) & 0x0F0F0F0Fu); };
    return v4i{c(b.qs.x), c(b.qs.y), c(b.qs.z), c(b.qs.w)};
  }
};

template <> struct QmmFmt<Q8_0> {
  static constexpr int BYTES = 8 * 34;
  struct Hdr {};
  struct Blk { u32x4 qs; uint32_t d; };  // int8 codes 16g .. 16g+15 of block j
  __device__ static Hdr hdr(const uint8_t*) { return Hdr{}; }
  __device__ static Blk blk(const uint8_t* sb, int j, int g) {
    unsigned short dh;
    __builtin_memcpy(&dh, sb + 34 * j, 2);
    return Blk{ld16(sb + 34 * j + 2 + 16 * g), dh};
  }
  template <int J> __device__ static double scale(const Hdr&, const Blk& b) { return (double)h2f(b.d); }
  template <int J> __device__ static v4i codes(const Blk& b, int /*g*/) {
    return v4i{(int)b.qs.x, (int)b.qs.y, (int)b.qs.z, (int)b.qs.w};
  }
};

template <> struct QmmFmt<Q6_K> {
  static constexpr int BYTES = 210;
  struct Hdr { u32x4 sc; uint32_t d; };
  // Block j = sub-blocks 2j (first 16 elements) and 2j+1; this lane's K-slice
  // g covers elements 8g..8g+7 of each: ql and qh bytes for l in those ranges.
  struct Blk { u32x2 l0, l1, h0, h1; };
  __device__ static Hdr hdr(const uint8_t* sb) {
    Hdr x;
    x.sc = ld16(sb + 192);
    unsigned short dh;
    __builtin_memcpy(&dh, sb + 208, 2);
    x.d = dh;
    return x;
  }
  __device__ static Blk blk(const uint8_t* sb, int j, int g) {
    const int h = j >> 2, g6 = j & 3;
    const uint8_t* ql = sb + 64 * h + 32 * (g6 & 1) + 8 * g;
    const uint8_t* qh = sb + 128 + 32 * h + 8 * g;
    return Blk{ld8(ql), ld8(ql + 16), ld8(qh), ld8(qh + 16)};
  }
  // int8 sub-scales of sub-blocks 2j, 2j+1
  template <int J> __device__ static void scales(const Hdr& x, int& s0, int& s1) {
    const uint32_t w = J < 2 ? x.sc.x : (J < 4 ? x.sc.y : (J < 6 ? x.sc.z : x.sc.w));
    s0 = (int)(int8_t)(w >> (16 * (J & 1)));
    s1 = (int)(int8_t)(w >> (16 * (J & 1) + 8));
  }
  // signed codes of sub-block 2j + half (8 bytes = this lane's K-slice)
  template <int J> __device__ static long codes(const Blk& b, int half) {
    constexpr int g6 = J & 3;
    const u32x2 lq = half ? b.l1 : b.l0, hq = half ? b.h1 : b.h0;
    uint32_t c[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      c[k] = q6k_signed(q6k_code<(g6 >= 2)>(lq[k], hq[k], g6 & 1));
    }
    return (long)((uint64_t)c[0] | ((uint64_t)c[1] << 32));
  }
};

// --------------------------------------------------------------- kernel
// Weight staging.  Each iteration the workgroup copies the superblocks it
// works on next -- superblock kp + KP*it of each of its QMM_BN weight rows,
// for every K slice kp -- into LDS with 16-byte chunk copies in which
// consecutive lanes take consecutive bytes of a row, so one copy instruction
// of a wave touches a few cache lines, where the MFMA operand layout (lane l
// <-> row l%32) would touch 32; the waves that share a K slice read the one
// copy.  A row's superblock keeps its own byte order at a pitch of its size
// rounded up to 16 bytes, so the format decoders read it as they read HBM.
// Q6_K rows are read 8 bytes per lane, 32 rows at once: a pitch of 58
// dwords (232 bytes) puts those 32 reads on 64 distinct banks, where the
// 16-byte multiple (224) would put rows r, r+8, r+16, r+24 on the same ones.
template <int T> constexpr int qmm_cpr() { return (Geom<T>::BYTES + 15) / 16; }  // 16-byte pieces per row
template <int T> constexpr int qmm_pitch() { return T == Q6_K ? 232 : 16 * qmm_cpr<T>(); }
template <int T, int KP> constexpr int qmm_stage_chunks() { return KP * QMM_BN * qmm_cpr<T>(); }
template <int T, int KP> constexpr int qmm_stage_regs() {  // 16-byte chunks each thread copies
  return (qmm_stage_chunks<T, KP>() + 64 * QMM_WAVES - 1) / (64 * QMM_WAVES);
}
// LDS: the per-wave fp64 activation scales of one superblock, then the
// weight stage; after the main loop the K-split partial sums reuse it.
constexpr int QMM_SCALE_BYTES = QMM_WAVES * 8 * 32 * 16;
template <int KP> constexpr int qmm_red_bytes() { return (QMM_WAVES - QMM_WAVES / KP) * QMM_NT * 16 * 64 * 8; }
template <int T, int KP> constexpr int qmm_stage_bytes() { return KP * QMM_BN * qmm_pitch<T>(); }
template <int T, int KP> constexpr int qmm_lds_bytes() {
  return QMM_SCALE_BYTES + qmm_stage_bytes<T, KP>() > qmm_red_bytes<KP>()
             ? QMM_SCALE_BYTES + qmm_stage_bytes<T, KP>()
             : qmm_red_bytes<KP>();
}

// Two workgroups (two waves per SIMD) per CU wherever the LDS allows it;
// the Q8_0 K-split-4 instance (a 272-byte-pitch stage) holds one, and so do
// the Q6_K K-split-4 instance (its 56 staging registers spill at two waves:
// 1024 x 4096 at M = 512 42 us at two, 37.6 at one) and the sub-block-sum
// dump (a test path: fewer spills at one wave).
template <int T, int KP, bool DUMP> constexpr int qmm_min_waves() {
  return !DUMP && !(T == Q6_K && KP == 4) && qmm_lds_bytes<T, KP>() <= 80 * 1024 ? 2 : 1;
}

template <int T> constexpr int qmm_ring() { return T == Q6_K ? 2 : 4; }  // A-operand ring: loads run ring-1 blocks ahead


template <int KP> constexpr int qmm_bm() { return 32 * QMM_WAVES / KP; }  // activation rows per workgroup

template <int T, int KP, bool DUMP>
__device__ __forceinline__ void qmm_split_tile(const uint8_t* __restrict__ W, int N, int K,
                                               const uint8_t* __restrict__ xq, int M, float* __restrict__ y,
                                               int32_t* __restrict__ isums, int m_tiles, int n_tiles) {
  static_assert(T != Q4_K, "Q4_K runs the 16x16 tile (qmm_q4k16_tile)");
  using F = QmmFmt<T>;
  constexpr int SUB = Geom<T>::SUB;
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int PITCH = qmm_pitch<T>();
  constexpr int CPR = qmm_cpr<T>();                    // chunks per staged row
  constexpr int CHUNKS = qmm_stage_chunks<T, KP>();
  constexpr int NCH = qmm_stage_regs<T, KP>();
  constexpr int QMM_RING = qmm_ring<T>();
  static_assert(8 % QMM_RING == 0, "ring slot of block j must not depend on the superblock");
  static_assert(QMM_WAVES % KP == 0, "K split must divide the waves");
  // Activation scales of this wave's 32 rows for its current superblock,
  // fp64: [wave][block][row].  Each wave reads only its own slice, so a
  // wave-level barrier orders the staging.
  __shared__ __align__(16) double lds_raw[qmm_lds_bytes<T, KP>() / 8];
  QmmDs(*const lds_ds)[8][32] = reinterpret_cast<QmmDs(*)[8][32]>(lds_raw);
  uint8_t* const lds_w = reinterpret_cast<uint8_t*>(lds_raw) + QMM_SCALE_BYTES;

  // XCD-aware tile order: workgroup id i runs on XCD i % 8; the m_tiles
  // workgroups that share a weight tile get ids with the same residue, so
  // they run on one XCD and read the weight tile from its L2.
  const int id = blockIdx.x;
  const int xcd = id % QMM_XCDS, local = id / QMM_XCDS;
  const int m_tile = local % m_tiles;
  const int n_tile = (local / m_tiles) * QMM_XCDS + xcd;
  if (n_tile >= n_tiles) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, c32 = lane & 31;
  const int kp = wave % KP, wq = wave / KP;
  const int nsb = K / QK, nq8 = K / Q8_BLOCK;
  const size_t row_bytes = (size_t)nsb * BYTES;
  const int m0 = m_tile * qmm_bm<KP>() + 32 * wq;
  const int n0 = n_tile * QMM_BN;

  // This lane's activation row (A operand and scale staging); rows past the
  // edge are clamped to the last one and never stored.
  const int ma = m0 + c32 < M ? m0 + c32 : M - 1;
  const uint8_t* xrow = xq + (size_t)ma * nq8 * Q8_BYTES;
  // This lane's staged weight rows (B operand) in K slice kp.
  const uint8_t* wl[QMM_NT];
#pragma unroll
  for (int t = 0; t < QMM_NT; ++t) wl[t] = lds_w + (size_t)(kp * QMM_BN + 32 * t + c32) * PITCH;
  QmmDs(*const stage)[32] = lds_ds[wave];
  // The Q6_K instance with four K slices (one wave per SIMD) keeps only D,
  // as fp32 (an fp16 value, exact): half the LDS bytes of its sixteen D
  // reads per block (v 1024 x 4096 at M = 512: 35.2 -> 32.3 us; with two
  // K slices the conversions cost what the bytes save).
  constexpr bool D32 = T == Q6_K && KP == 4;
  float(*const dstage)[32] = reinterpret_cast<float(*)[32]>(lds_ds[wave]);

  // Stage copy: chunk i = (K slice s, row r, 16-byte piece c); rows past N
  // are clamped to the last row, superblocks past the row to the last one
  // (in bounds, never used).  The loads are unconditional (threads past the
  // last chunk repeat it; only the LDS store is skipped), so no branch makes
  // the compiler wait for them before the compute.  The last piece of a 210-
  // or 136-byte superblock is read as the 16 bytes that end the superblock
  // and shifted down.
  auto stage_load = [&](int it, u32x4 (&breg)[NCH]) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int iu = tid + 64 * QMM_WAVES * u;
      const int i = iu < CHUNKS ? iu : CHUNKS - 1;
      const int s = i / (QMM_BN * CPR), rem = i % (QMM_BN * CPR);
      const int r = rem / CPR, c = rem % CPR;
      const int n = n0 + r < N ? n0 + r : N - 1;
      int bb = s + KP * it;
      bb = bb < nsb ? bb : nsb - 1;
      const uint8_t* sb = W + (size_t)n * row_bytes + (size_t)bb * BYTES;
      if constexpr (BYTES % 16 == 0) {
        breg[u] = ld16(sb + 16 * c);
      } else {
        constexpr int TAIL = BYTES % 16;
        const bool tail = c == CPR - 1;
        const u32x4 v = ld16(sb + (tail ? BYTES - 16 : 16 * c));
        if constexpr (TAIL == 8) {
          breg[u] = tail ? u32x4{v.z, v.w, 0u, 0u} : v;
        } else {
          static_assert(TAIL == 2, "tail piece of 2 or 8 bytes");
          breg[u] = tail ? u32x4{v.w >> 16, 0u, 0u, 0u} : v;
        }
      }
    }
  };
  auto stage_store = [&](const u32x4 (&breg)[NCH]) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int i = tid + 64 * QMM_WAVES * u;
      if (i < CHUNKS) {
        if constexpr (PITCH == 16 * CPR) {
          *reinterpret_cast<u32x4*>(lds_w + 16 * i) = breg[u];
        } else {  // padded rows: the piece lands 8-byte aligned
          const int sr = i / CPR, c = i % CPR;
          u32x2* dst = reinterpret_cast<u32x2*>(lds_w + sr * PITCH + 16 * c);
          dst[0] = u32x2{breg[u].x, breg[u].y};
          dst[1] = u32x2{breg[u].z, breg[u].w};
        }
      }
    }
  };
  // A operand of block j of superblock b (this lane's row and K-slice g).
  auto load_a = [&](int b, int j) {
    const uint8_t* xb = xrow + (size_t)(b * 8 + j) * Q8_BYTES + 4;
    if constexpr (T == Q6_K) {
      return ld16(xb + 16 * g);  // elements 16g .. 16g+15; see the exchange in the block loop
    } else {
      return ld16(xb + 16 * g);
    }
  };
  // Scales of row c32, blocks 4g..4g+3 of superblock b (raw fp16 pairs).
  auto load_ds = [&](int b, uint32_t* ds) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ds[u] = ld4(xrow + (size_t)(b * 8 + 4 * g + u) * Q8_BYTES);
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  double acc[QMM_NT][16];
#pragma unroll
  for (int t = 0; t < QMM_NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.0;

  // Every wave runs the same number of iterations (the workgroup barriers
  // need it); a wave whose K slice has run out skips the compute (with
  // K = 256 the second slice has no superblock at all, and its prologue
  // loads are clamped in bounds).
  const int nit = (nsb + KP - 1) / KP;
  const int b0 = kp < nsb ? kp : nsb - 1;
  u32x4 breg[NCH];
  stage_load(0, breg);
  uint32_t ds_next[4];
  load_ds(b0, ds_next);
  u32x4 ring[QMM_RING];
#pragma unroll
  for (int j = 0; j < QMM_RING - 1; ++j) ring[j] = load_a(b0, j);
  stage_store(breg);
  __syncthreads();

#pragma unroll 1
  for (int it = 0; it < nit; ++it) {
    const int b = kp + KP * it;
    const int bn = b + KP < nsb ? b + KP : nsb - 1;  // clamped: the last prefetch is redundant, in bounds
    const bool more = it + 1 < nit;                  // uniform over the workgroup
    stage_load(it + 1, breg);                        // lands while this superblock is computed
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if constexpr (D32) dstage[4 * g + u][c32] = h2f(ds_next[u] & 0xFFFFu);
      else stage[4 * g + u][c32] = QmmDs{(double)h2f(ds_next[u] & 0xFFFFu), (double)h2f(ds_next[u] >> 16)};
    load_ds(bn, ds_next);
    wave_sync();

    if (b < nsb) {
      typename F::Hdr hd[QMM_NT];
#pragma unroll
      for (int t = 0; t < QMM_NT; ++t) hd[t] = F::hdr(wl[t]);

      auto do_block = [&](auto JC) {
        constexpr int J = decltype(JC)::value;
        constexpr int JN = J + QMM_RING - 1;  // block whose A operand is fetched now
        // one block at a time: keeps the scheduler from hoisting the staged
        // operand reads of all eight blocks into registers at once
        __builtin_amdgcn_sched_barrier(0);
        ring[JN % QMM_RING] = JN < 8 ? load_a(b, JN) : load_a(bn, JN - 8);
        const u32x4 oa = ring[J % QMM_RING];
        typename F::Blk wb[QMM_NT];
#pragma unroll
        for (int t = 0; t < QMM_NT; ++t) wb[t] = F::blk(wl[t], J, g);
        if constexpr (T == Q6_K) {
          // The MFMA of sub-block 2J+h takes elements 16h + 8g .. 16h + 8g+7
          // from the lane of K-slice g.  This lane loaded elements 16g ..
          // 16g+15 in one 16-byte load, so the two lanes of a row (l, l+32)
          // trade halves: v_permlane32_swap exchanges the upper half-wave's
          // first 8 bytes with the lower half-wave's last 8, which leaves
          // sub-block 2J's slice in the first result and 2J+1's in the second.
          const auto xl = __builtin_amdgcn_permlane32_swap(oa.x, oa.z, false, false);
          const auto xh = __builtin_amdgcn_permlane32_swap(oa.y, oa.w, false, false);
          const long a0 = (long)((uint64_t)xl[0] | ((uint64_t)xh[0] << 32));
          const long a1 = (long)((uint64_t)xl[1] | ((uint64_t)xh[1] << 32));
          v16i I0[QMM_NT], I1[QMM_NT];
          int s0[QMM_NT], s1[QMM_NT];
          double d[QMM_NT];
#pragma unroll
          for (int t = 0; t < QMM_NT; ++t) {
            const v16i z = {0};
            I0[t] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a0, F::template codes<J>(wb[t], 0), z, 0, 0, 0);
            I1[t] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a1, F::template codes<J>(wb[t], 1), z, 0, 0, 0);
            F::template scales<J>(hd[t], s0[t], s1[t]);
            d[t] = (double)h2f(hd[t].d);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = mfma_row(r, g);
            const double D = D32 ? (double)dstage[J][i] : stage[J][i].d;
#pragma unroll
            for (int t = 0; t < QMM_NT; ++t) {
              const int P = q6k_pair(s0[t], I0[t][r], s1[t], I1[t][r]);  // exact int
              acc[t][r] = fma(d[t] * D, (double)P, acc[t][r]);     // exact product
              if (DUMP) {
                const int m = m0 + i, n = n0 + 32 * t + c32;
                if (m < M && n < N) {
                  int32_t* p = isums + ((size_t)m * N + n) * (K / SUB) + (size_t)b * (QK / SUB) + 2 * J;
                  p[0] = I0[t][r];
                  p[1] = I1[t][r];
                }
              }
            }
          }
        } else {
          const v4i a = v4i{(int)oa.x, (int)oa.y, (int)oa.z, (int)oa.w};
          v16i I[QMM_NT];
          double w[QMM_NT];
#pragma unroll
          for (int t = 0; t < QMM_NT; ++t) {
            const v16i z = {0};
            I[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, F::template codes<J>(wb[t], g), z, 0, 0, 0);
            w[t] = F::template scale<J>(hd[t], wb[t]);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int i = mfma_row(r, g);
            const QmmDs e = stage[J][i];
#pragma unroll
            for (int t = 0; t < QMM_NT; ++t) {
              acc[t][r] = fma(w[t] * e.d, (double)I[t][r], acc[t][r]);  // exact product
              if (DUMP) {
                const int m = m0 + i, n = n0 + 32 * t + c32;
                if (m < M && n < N)
                  isums[((size_t)m * N + n) * (K / SUB) + (size_t)b * (QK / SUB) + J] = I[t][r];
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
    }
    if (more) {
      __syncthreads();  // every wave has read this iteration's staged weights
      stage_store(breg);
      __syncthreads();
    }
  }

  if constexpr (KP > 1) {
    // Partial sums of K slices 1..KP-1 go through LDS; slice 0 adds them in
    // slice order and stores.
    __syncthreads();  // every wave is done with its scale and weight staging
    double* red = lds_raw;
    auto slot = [&](int q, int k, int t, int r) {
      return ((((q * (KP - 1) + (k - 1)) * QMM_NT + t) * 16 + r) * 64) + lane;
    };
    if (kp > 0) {
#pragma unroll
      for (int t = 0; t < QMM_NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) red[slot(wq, kp, t, r)] = acc[t][r];
    }
    __syncthreads();
    if (kp > 0) return;
#pragma unroll 1
    for (int k = 1; k < KP; ++k)
#pragma unroll
      for (int t = 0; t < QMM_NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] += red[slot(wq, k, t, r)];
  }

#pragma unroll
  for (int t = 0; t < QMM_NT; ++t) {
    const int n = n0 + 32 * t + c32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + mfma_row(r, g);
      if (m < M && n < N) y[(size_t)m * N + n] = (float)acc[t][r];
    }
  }
}

// ------------------------------------------------------ Q4_K, 16x16 tiles
// The same workgroup, K split and weight staging as the tile above, but the
// block dots come from v_mfma_i32_16x16x32_i8 on 16 x 16 tiles (a wave's 32
// activation rows x 64 weight rows are 2 x 4 of them), whose result layout
// lets the Q4_K min term -dmin*m_j*S run on the fp64 matrix cores instead of
// the VALU: per superblock and tile, two v_mfma_f64_16x16x4_f64 add
// sum over blocks j of S(m, j) * (-dmin*m_j)(n) straight into the fp64
// accumulators (every product exact in fp64, as in the VALU form; only the
// order of the fp64 additions differs).  The VALU keeps d*sc_j*D*I per block
// and output: one product of the two exact scales, the conversion of I and
// one fma.  The weight scales d*sc_j and -dmin*m_j of the wave's 64 rows are
// unpacked once per superblock into a per-wave fp64 table.
//
// Lane layouts (measured on gfx950), g4 = lane / 16, c16 = lane % 16:
//   v_mfma_i32_16x16x32_i8: A = row c16, bytes 8*g4 .. 8*g4+7 of K; B =
//   column c16, same K bytes; result v of the lane = D[4*g4 + v][c16].
//   v_mfma_f64_16x16x4_f64: A = row c16, k = g4; B = column c16, k = g4;
//   result v of the lane = D[g4 + 4*v][c16].
// So the f64 A operand of lane c16 carries activation row qf_row(c16) =
// 4*(c16 % 4) + c16 / 4, which puts result v of the lane on row 4*g4 + v,
// where the integer tile keeps it.
typedef double v4d __attribute__((ext_vector_type(4)));
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int qf_row(int c16) { return 4 * (c16 & 3) + (c16 >> 2); }

struct QfW { double w, mn; };  // d*sc_j and -dmin*m_j of one weight row and block

template <int KP> constexpr int qf_lds_bytes() {
  // per-wave D, S tables [8][32] fp64, the weight stage, per-wave weight scale tables [8][64]
  return QMM_SCALE_BYTES + qmm_stage_bytes<Q4_K, KP>() + QMM_WAVES * 8 * 64 * 16 > qmm_red_bytes<KP>()
             ? QMM_SCALE_BYTES + qmm_stage_bytes<Q4_K, KP>() + QMM_WAVES * 8 * 64 * 16
             : qmm_red_bytes<KP>();
}

template <int KP, bool DUMP>
__device__ __forceinline__ void qmm_q4k16_tile(const uint8_t* __restrict__ W, int N, int K,
                                               const uint8_t* __restrict__ xq, int M, float* __restrict__ y,
                                               int32_t* __restrict__ isums, int m_tiles, int n_tiles) {
  constexpr int T = Q4_K;
  constexpr int BYTES = Geom<T>::BYTES;
  constexpr int PITCH = qmm_pitch<T>();
  constexpr int CPR = qmm_cpr<T>();
  constexpr int CHUNKS = qmm_stage_chunks<T, KP>();
  constexpr int NCH = qmm_stage_regs<T, KP>();
  constexpr int RING = 4;
  static_assert(PITCH == 16 * CPR, "unpadded Q4_K stage");
  __shared__ __align__(16) double lds_raw[qf_lds_bytes<KP>() / 8];
  uint8_t* const lds_w = reinterpret_cast<uint8_t*>(lds_raw) + QMM_SCALE_BYTES;

  const int id = blockIdx.x;
  const int xcd = id % QMM_XCDS, local = id / QMM_XCDS;
  const int m_tile = local % m_tiles;
  const int n_tile = (local / m_tiles) * QMM_XCDS + xcd;
  if (n_tile >= n_tiles) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, c32 = lane & 31, g4 = lane >> 4, c16 = lane & 15;
  const int kp = wave % KP, wq = wave / KP;
  const int nsb = K / QK, nq8 = K / Q8_BLOCK;
  const size_t row_bytes = (size_t)nsb * BYTES;
  const int m0 = m_tile * qmm_bm<KP>() + 32 * wq;
  const int n0 = n_tile * QMM_BN;

  // Per-wave tables: activation D and S of the wave's 32 rows, [block][row];
  // weight scales of its 64 rows, [block][row].
  double(*const Dt)[32] = reinterpret_cast<double(*)[32]>(lds_raw + wave * 512);
  double(*const St)[32] = reinterpret_cast<double(*)[32]>(lds_raw + wave * 512 + 256);
  QfW(*const Wt)[64] = reinterpret_cast<QfW(*)[64]>(
      reinterpret_cast<uint8_t*>(lds_raw) + QMM_SCALE_BYTES + qmm_stage_bytes<T, KP>() + wave * 8 * 64 * 16);

  // Activation rows of this lane: A operand rows 16*tm + c16 (clamped to the
  // last row past M; never stored) and the scale staging row c32.
  const uint8_t* xr[2];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int m = m0 + 16 * tm + c16 < M ? m0 + 16 * tm + c16 : M - 1;
    xr[tm] = xq + (size_t)m * nq8 * Q8_BYTES;
  }
  const int ms = m0 + c32 < M ? m0 + c32 : M - 1;
  const uint8_t* xs = xq + (size_t)ms * nq8 * Q8_BYTES;
  // Weight rows of this lane in K slice kp: B operand rows 16*tn + c16, and
  // row `lane` for the scale table.
  const uint8_t* wl[4];
#pragma unroll
  for (int tn = 0; tn < 4; ++tn) wl[tn] = lds_w + (size_t)(kp * QMM_BN + 16 * tn + c16) * PITCH;
  const uint8_t* wh = lds_w + (size_t)(kp * QMM_BN + lane) * PITCH;

  auto stage_load = [&](int it, u32x4 (&breg)[NCH]) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int iu = tid + 64 * QMM_WAVES * u;
      const int i = iu < CHUNKS ? iu : CHUNKS - 1;
      const int sl = i / (QMM_BN * CPR), rem = i % (QMM_BN * CPR);
      const int r = rem / CPR, c = rem % CPR;
      const int n = n0 + r < N ? n0 + r : N - 1;
      int bb = sl + KP * it;
      bb = bb < nsb ? bb : nsb - 1;
      breg[u] = ld16(W + (size_t)n * row_bytes + (size_t)bb * BYTES + 16 * c);
    }
  };
  auto stage_store = [&](const u32x4 (&breg)[NCH]) {
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int i = tid + 64 * QMM_WAVES * u;
      if (i < CHUNKS) *reinterpret_cast<u32x4*>(lds_w + 16 * i) = breg[u];
    }
  };
  // A operand of block j of superblock b: 8 bytes of rows 16*tm + c16.
  auto load_a = [&](int b, int j) {
    const size_t o = (size_t)(b * 8 + j) * Q8_BYTES + 4 + 8 * g4;
    const u32x2 a0 = ld8(xr[0] + o), a1 = ld8(xr[1] + o);
    return u32x4{a0.x, a0.y, a1.x, a1.y};
  };
  auto load_ds = [&](int b, uint32_t* ds) {
#pragma unroll
    for (int u = 0; u < 4; ++u) ds[u] = ld4(xs + (size_t)(b * 8 + 4 * g + u) * Q8_BYTES);
  };
  auto wave_sync = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  v4d acc[2][4];
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = v4d{0.0, 0.0, 0.0, 0.0};

  const int nit = (nsb + KP - 1) / KP;
  const int b0 = kp < nsb ? kp : nsb - 1;
  u32x4 breg[NCH];
  stage_load(0, breg);
  uint32_t ds_next[4];
  load_ds(b0, ds_next);
  u32x4 ring[RING];
#pragma unroll
  for (int j = 0; j < RING - 1; ++j) ring[j] = load_a(b0, j);
  stage_store(breg);
  __syncthreads();

#pragma unroll 1
  for (int it = 0; it < nit; ++it) {
    const int b = kp + KP * it;
    const int bn = b + KP < nsb ? b + KP : nsb - 1;
    const bool more = it + 1 < nit;
    stage_load(it + 1, breg);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      Dt[4 * g + u][c32] = (double)h2f(ds_next[u] & 0xFFFFu);
      St[4 * g + u][c32] = (double)h2f(ds_next[u] >> 16);
    }
    load_ds(bn, ds_next);
    {  // weight scales of row `lane`, all eight blocks
      const u32x4 h = ld16(wh);
      const float dw = h2f(h.x), dm = h2f(h.x >> 16);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t sc, mm;
        q4k_scale_min(h, j, sc, mm);
        Wt[j][lane] = QfW{(double)(dw * (float)sc), -(double)(dm * (float)mm)};
      }
    }
    wave_sync();

    if (b < nsb) {
      // The drain scales of block J (weight scales d*sc_J of the lane's four
      // weight rows, activation D of its eight activation rows) are read
      // from the tables one block ahead, after block J-1's operand reads,
      // so that their LDS latency overlaps block J-1's MFMAs and drains.
      struct Sc { double w[4], dv[2][4]; };
      auto load_sc = [&](int J, Sc& sc) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) sc.w[tn] = Wt[J][16 * tn + c16].w;
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
          const double* dp = &Dt[J][16 * tm + 4 * g4];
#pragma unroll
          for (int v = 0; v < 4; ++v) sc.dv[tm][v] = dp[v];
        }
      };
      Sc scs[2];
      load_sc(0, scs[0]);
      auto do_block = [&](auto JC) {
        constexpr int J = decltype(JC)::value;
        constexpr int JN = J + RING - 1;
        __builtin_amdgcn_sched_barrier(0);
        ring[JN % RING] = JN < 8 ? load_a(b, JN) : load_a(bn, JN - 8);
        const u32x4 oa = ring[J % RING];
        const long a0 = (long)((uint64_t)oa.x | ((uint64_t)oa.y << 32));
        const long a1 = (long)((uint64_t)oa.z | ((uint64_t)oa.w << 32));
        u32x2 q[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) q[tn] = *reinterpret_cast<const u32x2*>(wl[tn] + 16 + 32 * (J >> 1) + 8 * g4);
        constexpr int kc = J / 4, tmm = (J / 2) % 2;
        const double sa = St[4 * kc + g4][16 * tmm + qf_row(c16)];
        double smn[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) smn[e] = Wt[4 * kc + g4][16 * (2 * (J % 2) + e) + c16].mn;
        if constexpr (J < 7) load_sc(J + 1, scs[(J + 1) % 2]);
        const Sc& sc = scs[J % 2];
        v4i_t I[2][4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
          constexpr int sh = (J & 1) ? 4 : 0;
          const long bq = (long)((uint64_t)((q[tn].x >> sh) & 0x0F0F0F0Fu) |
                                 ((uint64_t)((q[tn].y >> sh) & 0x0F0F0F0Fu) << 32));
          const v4i_t z = {0, 0, 0, 0};
          I[0][tn] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a0, bq, z, 0, 0, 0);
          I[1][tn] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a1, bq, z, 0, 0, 0);
        }
        // two of the superblock's sixteen min-term MFMAs: blocks 4*kc + g4 of tile (tmm, tn)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int tn = 2 * (J % 2) + e;
          acc[tmm][tn] = __builtin_amdgcn_mfma_f64_16x16x4f64(sa, smn[e], acc[tmm][tn], 0, 0, 0);
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm) {
#pragma unroll
          for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              acc[tm][tn][v] = fma(sc.w[tn] * sc.dv[tm][v], (double)I[tm][tn][v], acc[tm][tn][v]);  // exact product
              if (DUMP) {
                const int m = m0 + 16 * tm + 4 * g4 + v, n = n0 + 16 * tn + c16;
                if (m < M && n < N) isums[((size_t)m * N + n) * (K / 32) + (size_t)b * 8 + J] = I[tm][tn][v];
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
    }
    if (more) {
      __syncthreads();
      stage_store(breg);
      __syncthreads();
    }
  }

  if constexpr (KP > 1) {
    __syncthreads();
    double* red = lds_raw;
    auto slot = [&](int q, int k, int tm, int tn, int v) {
      return (((((q * (KP - 1) + (k - 1)) * 2 + tm) * 4 + tn) * 4 + v) * 64) + lane;
    };
    if (kp > 0) {
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[slot(wq, kp, tm, tn, v)] = acc[tm][tn][v];
    }
    __syncthreads();
    if (kp > 0) return;
#pragma unroll 1
    for (int k = 1; k < KP; ++k)
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[tm][tn][v] += red[slot(wq, k, tm, tn, v)];
  }

#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
      const int n = n0 + 16 * tn + c16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * tm + 4 * g4 + v;
        if (m < M && n < N) y[(size_t)m * N + n] = (float)acc[tm][tn][v];
      }
    }
}

template <int T, int KP, bool DUMP> constexpr int qmm_occupancy() {
  if constexpr (T == Q4_K) return !DUMP && qf_lds_bytes<KP>() <= 80 * 1024 ? 2 : 1;
  else return qmm_min_waves<T, KP, DUMP>();
}

template <int T, int KP, bool DUMP>
__global__ __launch_bounds__(64 * QMM_WAVES, (qmm_occupancy<T, KP, DUMP>())) void qmm_mfma_kernel(
    const uint8_t* __restrict__ W, int N, int K, const uint8_t* __restrict__ xq, int M,
    float* __restrict__ y, int32_t* __restrict__ isums, int m_tiles, int n_tiles) {
  if constexpr (T == Q4_K) qmm_q4k16_tile<KP, DUMP>(W, N, K, xq, M, y, isums, m_tiles, n_tiles);
  else qmm_split_tile<T, KP, DUMP>(W, N, K, xq, M, y, isums, m_tiles, n_tiles);
}

// K split: 2 or 4 waves per output tile, from N and K only (never M), so
// that an output's value does not depend on M.  Measured on MI355X at M = 512
// (Qwen3-8B and hidden-5120 shapes, occupancy two waves per SIMD): two slices
// beat one and four for N > 2048; four slices win for N <= 2048, where the
// grid is otherwise too small to fill 256 CUs.  With fewer superblocks than
// slices the extra waves idle (K = 256: one superblock, two slices).
inline int qmm_ksplit(int N, int K) {
  const int nsb = K / QK;
  int kp = N <= 2048 ? 4 : 2;
  if (kp > nsb) kp = 2;
  return kp;
}

template <int T, int KP, bool DUMP>
inline int launch_qmm_kp(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                         int32_t* isums, hipStream_t s) {
  const int m_tiles = (M + qmm_bm<KP>() - 1) / qmm_bm<KP>();
  const int n_tiles = (N + QMM_BN - 1) / QMM_BN;
  const long groups = (long)(n_tiles + QMM_XCDS - 1) / QMM_XCDS;
  const long grid = (long)QMM_XCDS * m_tiles * groups;
  if (grid > 0x7FFFFFFFL) return -1;
  hipLaunchKernelGGL((qmm_mfma_kernel<T, KP, DUMP>), dim3((unsigned)grid), dim3(64 * QMM_WAVES), 0, s,
                     W, N, K, xq, M, y, isums, m_tiles, n_tiles);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int T, bool DUMP>
inline int launch_qmm_t(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                        int32_t* isums, hipStream_t s) {
  if (qmm_ksplit(N, K) == 2) return launch_qmm_kp<T, 2, DUMP>(W, N, K, xq, M, y, isums, s);
  return launch_qmm_kp<T, 4, DUMP>(W, N, K, xq, M, y, isums, s);
}

}  // namespace qdot
