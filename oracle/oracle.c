/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the block-quantized
 * integer-dot matmul (Q8_1 activations x Q4_K / Q6_K / IQ4_XS / Q4_0 / Q8_0
 * weights -> fp32), and for one decode step of attention over a 4-bit KV
 * cache (oracle_attn_decode_kv4, at the end of this file).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library) never calls it, shares no code, header, table or constant with
 * it, and must fail loudly if its own extension is missing.
 *
 * What it computes, and where the pages say so:
 *   - xLLM v0.7 dev log (developer.cloud.tencent.com.cn/article/2739032),
 *     section 1 "background": the matmul runs integer dot products directly on
 *     the raw Q4_K / Q6_K quantized weights and only then produces fp32, instead
 *     of dequantizing the weights to fp32 first.
 *   - same page, section B1.3: the Q8 activation quantization adds about 0.5 %
 *     RMS noise against an unquantized fp32 SGEMV and keeps the argmax.
 *   - V100TPS operations log (agent-report.daedalus.work), 2026-08-12 entry
 *     "batch kernel locked to Q4_0": an IQ4_XS 32-element sub-block is laid out
 *     like a Q4_0 block (low nibbles are elements 0-15, high nibbles 16-31), its
 *     scale is d*(ls-32) and its values come from the kvalues_iq4nl lookup.
 *   - Kestrel_VLLM #18 (wsisp.com), section 5 "limits": the block dot is an
 *     exact int32 sum inside each block; the scales are applied afterwards.
 *
 * The pages print neither the Q4_K / Q6_K / Q8_1 bit layouts, nor the IQ4_NL
 * codebook values, nor the activation quantizer's rounding.  The readings used
 * here (plain GGUF layouts, a placeholder codebook, round-half-away quantizer)
 * are listed one by one at each function.
 *
 * Arithmetic: integer sums in int64; every scale product is formed in fp64 in
 * an order where each partial product is exact (fp16 has 11 significant bits,
 * so d*sc*D*I needs at most 11+6+11+17 = 45 bits < 53); the terms are summed in
 * fp64 in K order and the result is rounded once to fp32 (round to nearest
 * even).  Built with -O1 -ffp-contract=off, no fast-math, no SIMD intrinsics.
 *
 * Threads: the matmul and sub-block-sum loops run their independent outputs
 * on several host threads (OpenMP, when built with it; oracle_set_threads
 * picks the count).  Each output is still computed by one thread with exactly
 * the operations and order written below, so the results do not depend on
 * the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_Q4_K 1
#define OR_Q6_K 2
#define OR_IQ4_XS 3
#define OR_Q4_0 4
#define OR_Q8_0 5

#define OR_QK 256        /* weights per superblock (Q4_0 / Q8_0: a group of
                            eight consecutive 32-weight blocks)            */
#define OR_Q8_BLOCK 32   /* activations per Q8_1 block                   */
#define OR_Q8_BYTES 36   /* fp16 d, fp16 s, 32 x int8                    */

/* IQ4_NL-style codebook.  PLACEHOLDER: the pages name kvalues_iq4nl but do
 * not print its values, and no copy of the format's table is available here.
 * This stand-in is strictly increasing and non-uniform:
 *     v_i = round_half_away(-127 + 240 * (i/15)^1.4),  i = 0..15.
 * Compatibility with real IQ4_XS files is therefore unpinned. */
static const int oracle_iq4nl_codebook[16] = {
    -127, -122, -113, -102, -89, -75, -60, -44,
    -27,  -10,  9,    28,   49,  69,  91,  113};

const int *oracle_codebook(void) { return oracle_iq4nl_codebook; }

/* ---------------------------------------------------------------- binary16 */

/* Exact decode of an IEEE binary16 bit pattern, subnormals included. */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);               /* 0.f * 2^-14 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);   /* 1.f * 2^(e-15) */
  return sign ? -v : v;
}

/* Round a double to the nearest binary16, ties to even (IEEE default).
 * nearbyint() uses the current rounding mode, which is round-to-nearest-even
 * unless someone changed it; ldexp() is exact. */
uint16_t oracle_double_to_half(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (isnan(v)) return 0x7E00u;
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u); /* 65520 is the tie above 65504 */
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: value = m * 2^-24, m in [0, 1024] (1024 = min normal) */
    double m = nearbyint(ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)m);
  }
  int e;
  frexp(a, &e);                          /* a in [2^(e-1), 2^e)            */
  double m = nearbyint(ldexp(a, 11 - e)); /* 11 significant bits: [1024,2048] */
  int E = e - 1;
  if (m == 2048.0) { m = 1024.0; E += 1; }
  return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)m - 1024));
}

/* Host threads used by the loops over outputs below (1 when built without
 * OpenMP).  n < 1 restores the OpenMP default this process started with
 * (OMP_NUM_THREADS, else all cores). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  static int initial = 0;
  if (initial == 0) initial = omp_get_max_threads();
  omp_set_num_threads(n >= 1 ? n : initial);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static uint16_t rd16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }
static void wr16(uint8_t *p, uint16_t v) { p[0] = (uint8_t)(v & 255); p[1] = (uint8_t)(v >> 8); }

/* --------------------------------------------------------------- Q8_1 side */

/* Q8_1 activation quantizer (the pages' quantize_q8_1; V100TPS log, 2026-08-12
 * entries on ggml_mul_mat_a8, which launches it ahead of the matmul).
 * Readings (the pages are silent on the rounding):
 *   amax = max |x_i| over the 32-element block, in fp32;
 *   d32  = amax / 127 (one correctly rounded fp32 division);
 *   q_i  = roundf(x_i / d32) (fp32 division, ties away from zero), clamped to
 *          [-127, 127]; all zero when amax == 0;
 *   D    = binary16(d32), round to nearest even;
 *   S    = binary16(D * sum_i q_i); the product is exact in fp32 (11 + 12 bits),
 *          so S takes exactly one rounding.
 * Block bytes: D (little endian) at 0, S at 2, q_0..q_31 at 4..35.
 * Rows: x is [M][K] row-major fp32; out is [M][K/32] blocks of 36 bytes. */
void oracle_quantize_q8_1(const float *x, int64_t M, int64_t K, uint8_t *out) {
  int64_t nblk = K / OR_Q8_BLOCK;
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t b = 0; b < nblk; ++b) {
      const float *xb = x + m * K + b * OR_Q8_BLOCK;
      uint8_t *ob = out + (m * nblk + b) * OR_Q8_BYTES;
      float amax = 0.0f;
      for (int i = 0; i < OR_Q8_BLOCK; ++i) {
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      int sumq = 0;
      int8_t q[OR_Q8_BLOCK];
      float d32 = 0.0f;
      if (amax == 0.0f) {
        memset(q, 0, sizeof q);
      } else {
        d32 = amax / 127.0f;
        for (int i = 0; i < OR_Q8_BLOCK; ++i) {
          float r = roundf(xb[i] / d32);
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          q[i] = (int8_t)r;
          sumq += q[i];
        }
      }
      uint16_t D = oracle_double_to_half((double)d32);
      double Dd = oracle_half_to_double(D);
      uint16_t S = oracle_double_to_half(Dd * (double)sumq);
      wr16(ob, D);
      wr16(ob + 2, S);
      memcpy(ob + 4, q, OR_Q8_BLOCK);
    }
  }
}

/* RMSNorm of each row (the producer of the Q8_1 activations of the Q/K/V and
 * gate/up projections: the xLLM engine quantizes the normalized input into
 * one shared buffer, d_xn_q8, section C.1).  Kestrel_VLLM #18, section 3.6
 * (the CPU-order RMSNorm kernel and the first row of its table) fixes the
 * numerics, including the order of the sum of squares:
 *   - each group of 8 consecutive elements e_0..e_7 is summed as a
 *     horizontal 8-wide sum: lo_k = e_k^2 + e_(k+4)^2 for k < 4, then
 *     (lo_0 + lo_1) + (lo_2 + lo_3);
 *   - the group sums are added one after the other, left to right, into a
 *     single fp32 accumulator that starts at zero (ss = ss + group);
 *   - r = 1.0f / sqrtf(ss / K + eps), a correctly rounded division and
 *     square root, not an rsqrt approximation;
 *   - out_i = (x_i * r) * w_i.
 * Every operation is one fp32 operation (built with -ffp-contract=off, so
 * nothing is fused).  K is a multiple of 32 here, so no element is left over
 * after the last group of 8.
 * xn is [M][K] fp32; ss[m] receives the row's sum of squares. */
void oracle_rmsnorm(const float *x, const float *w, float eps, int64_t M, int64_t K, float *xn,
                    float *ss) {
  for (int64_t m = 0; m < M; ++m) {
    const float *xr = x + m * K;
    float acc = 0.0f;
    for (int64_t g = 0; g + 8 <= K; g += 8) {
      const float *e = xr + g;
      float lo[4];
      for (int k = 0; k < 4; ++k) {
        float s0 = e[k] * e[k];
        float s1 = e[k + 4] * e[k + 4];
        lo[k] = s0 + s1;
      }
      float s01 = lo[0] + lo[1];
      float s23 = lo[2] + lo[3];
      float grp = s01 + s23;
      acc = acc + grp;
    }
    float mean = acc / (float)K;
    float r = 1.0f / sqrtf(mean + eps);
    ss[m] = acc;
    for (int64_t k = 0; k < K; ++k) {
      float a = xr[k] * r;
      xn[m * K + k] = a * w[k];
    }
  }
}

/* Exact dequantization of Q8_1 blocks: xhat[m][k] = D * q. */
void oracle_dequant_q8_1(const uint8_t *xq, int64_t M, int64_t K, double *xhat) {
  int64_t nblk = K / OR_Q8_BLOCK;
  for (int64_t m = 0; m < M; ++m)
    for (int64_t b = 0; b < nblk; ++b) {
      const uint8_t *blk = xq + (m * nblk + b) * OR_Q8_BYTES;
      double D = oracle_half_to_double(rd16(blk));
      for (int i = 0; i < OR_Q8_BLOCK; ++i)
        xhat[m * K + b * OR_Q8_BLOCK + i] = D * (double)(int8_t)blk[4 + i];
    }
}

/* ------------------------------------------------------- weight superblocks */

/* One decoded superblock: 256 integer weight codes, grouped in sub-blocks of
 * `sublen` elements; w = scale[j] * code - minv[j] for sub-block j.  The scale
 * and min are kept as (fp16 value) x (small integer) so that products stay
 * exact. */
typedef struct {
  int sublen;        /* 32 (Q4_K, IQ4_XS) or 16 (Q6_K)                  */
  int nsub;          /* 8 or 16                                         */
  int code[OR_QK];   /* Q4_K: 0..15; Q6_K: -32..31; IQ4_XS: codebook    */
  double d;          /* superblock scale                                */
  double dmin;       /* Q4_K only, else 0                               */
  int sc[16];        /* integer sub-block scale multiplier              */
  int mn[16];        /* Q4_K integer sub-block min multiplier, else 0   */
  double dj[16];     /* scale of sub-block j's code sum: d*sc_j (exact) */
  double mj[16];     /* Q4_K min of sub-block j: dmin*m_j (exact), else 0 */
} oracle_sb;

static int block_bytes(int type) {
  switch (type) {
    case OR_Q4_K: return 144;
    case OR_Q6_K: return 210;
    case OR_IQ4_XS: return 136;
    case OR_Q4_0: return 8 * 18;
    case OR_Q8_0: return 8 * 34;
    default: return 0;
  }
}

/* Q4_K superblock (144 B).  Reading (plain GGUF layout; the pages name the
 * format but print no layout):
 *   bytes 0-1 d, 2-3 dmin (binary16, little endian), 4-15 scales[12],
 *   16-143 qs[128].
 *   Sub-block j (32 elements) has a 6-bit scale sc_j and 6-bit min m_j:
 *     j < 4 : sc_j = scales[j] & 63,  m_j = scales[j+4] & 63
 *     j >= 4: sc_j = (scales[j+4] & 15) | ((scales[j-4] >> 6) << 4)
 *             m_j  = (scales[j+4] >> 4) | ((scales[j]   >> 6) << 4)
 *   Byte qs[32c + l] (c < 4, l < 32) holds element 64c + l in its low nibble
 *   and element 64c + 32 + l in its high nibble.
 *   Weight: w = d * sc_j * q - dmin * m_j. */
static void decode_q4_k(const uint8_t *p, oracle_sb *s) {
  s->sublen = 32;
  s->nsub = 8;
  s->d = oracle_half_to_double(rd16(p));
  s->dmin = oracle_half_to_double(rd16(p + 2));
  const uint8_t *sc = p + 4;
  for (int j = 0; j < 8; ++j) {
    if (j < 4) {
      s->sc[j] = sc[j] & 63;
      s->mn[j] = sc[j + 4] & 63;
    } else {
      s->sc[j] = (sc[j + 4] & 15) | ((sc[j - 4] >> 6) << 4);
      s->mn[j] = (sc[j + 4] >> 4) | ((sc[j] >> 6) << 4);
    }
  }
  const uint8_t *qs = p + 16;
  for (int c = 0; c < 4; ++c)
    for (int l = 0; l < 32; ++l) {
      uint8_t byte = qs[32 * c + l];
      s->code[64 * c + l] = byte & 15;
      s->code[64 * c + 32 + l] = byte >> 4;
    }
}

/* Q6_K superblock (210 B).  Reading (plain GGUF layout):
 *   bytes 0-127 ql, 128-191 qh, 192-207 scales (int8), 208-209 d.
 *   For element e: h = e / 128, g = (e % 128) / 32, l = e % 32;
 *     low 4 bits  = ql[64h + 32*(g & 1) + l], shifted right by 4 when g >= 2;
 *     high 2 bits = (qh[32h + l] >> (2g)) & 3;
 *     code = (low | high << 4) - 32, in [-32, 31].
 *   Sub-block t = e / 16 (16 elements) has the int8 scale scales[t].
 *   Weight: w = d * scales[t] * code. */
static void decode_q6_k(const uint8_t *p, oracle_sb *s) {
  s->sublen = 16;
  s->nsub = 16;
  const uint8_t *ql = p, *qh = p + 128;
  const int8_t *scl = (const int8_t *)(p + 192);
  s->d = oracle_half_to_double(rd16(p + 208));
  s->dmin = 0.0;
  for (int t = 0; t < 16; ++t) {
    s->sc[t] = scl[t];
    s->mn[t] = 0;
  }
  for (int e = 0; e < OR_QK; ++e) {
    int h = e / 128, g = (e % 128) / 32, l = e % 32;
    int low = ql[64 * h + 32 * (g & 1) + l];
    if (g >= 2) low >>= 4;
    low &= 15;
    int high = (qh[32 * h + l] >> (2 * g)) & 3;
    s->code[e] = (low | (high << 4)) - 32;
  }
}

/* IQ4_XS superblock (136 B).  Layout of the nibbles and the scale rule from the
 * V100TPS log, 2026-08-12 "batch kernel locked to Q4_0" (low nibbles are
 * elements 0-15 of each 32-element sub-block, high nibbles 16-31; scale
 * d*(ls-32); value from the codebook).  The scale bit split is a reading:
 *   bytes 0-1 d, 2-3 scales_h (u16, little endian), 4-7 scales_l, 8-135 qs.
 *   ls_j = ((scales_l[j/2] >> (4*(j%2))) & 15) | (((scales_h >> (2j)) & 3) << 4)
 *   Byte qs[16j + i] (i < 16) holds element 32j + i (low nibble) and element
 *   32j + 16 + i (high nibble).
 *   Weight: w = d * (ls_j - 32) * codebook[nibble]. */
static void decode_iq4_xs(const uint8_t *p, oracle_sb *s) {
  s->sublen = 32;
  s->nsub = 8;
  s->d = oracle_half_to_double(rd16(p));
  s->dmin = 0.0;
  unsigned sh = rd16(p + 2);
  const uint8_t *sl = p + 4, *qs = p + 8;
  for (int j = 0; j < 8; ++j) {
    int ls = ((sl[j / 2] >> (4 * (j % 2))) & 15) | (((sh >> (2 * j)) & 3) << 4);
    s->sc[j] = ls - 32;
    s->mn[j] = 0;
    for (int i = 0; i < 16; ++i) {
      uint8_t byte = qs[16 * j + i];
      s->code[32 * j + i] = oracle_iq4nl_codebook[byte & 15];
      s->code[32 * j + 16 + i] = oracle_iq4nl_codebook[byte >> 4];
    }
  }
}

/* Q4_0 blocks (18 B per 32 weights), eight per 256-weight group.  The V100TPS
 * log (2026-08-12 entries) states the layout this oracle follows: a Q4_0 block
 * holds four 32-bit words of nibbles, low nibbles are elements 0-15 and high
 * nibbles elements 16-31, one scale d per block, value q - 8.  Reading for the
 * byte order (plain GGUF): bytes 0-1 d (binary16), 2-17 qs[16]; byte qs[i]
 * holds element i (low nibble) and element 16 + i (high nibble).
 *   Weight: w = d * (q - 8). */
static void decode_q4_0(const uint8_t *p, oracle_sb *s) {
  s->sublen = 32;
  s->nsub = 8;
  s->d = 1.0;
  s->dmin = 0.0;
  for (int j = 0; j < 8; ++j) {
    const uint8_t *blk = p + 18 * j;
    s->sc[j] = 1;
    s->mn[j] = 0;
    s->dj[j] = oracle_half_to_double(rd16(blk));
    s->mj[j] = 0.0;
    for (int i = 0; i < 16; ++i) {
      s->code[32 * j + i] = (blk[2 + i] & 15) - 8;
      s->code[32 * j + 16 + i] = (blk[2 + i] >> 4) - 8;
    }
  }
}

/* Q8_0 blocks (34 B per 32 weights), eight per 256-weight group.  The pages
 * name the 34-byte Q8_0 block (xLLM log, Phase B3/B4) without its layout;
 * reading (plain GGUF): bytes 0-1 d (binary16), 2-33 qs[32] (int8), element i
 * = qs[i].
 *   Weight: w = d * q. */
static void decode_q8_0(const uint8_t *p, oracle_sb *s) {
  s->sublen = 32;
  s->nsub = 8;
  s->d = 1.0;
  s->dmin = 0.0;
  for (int j = 0; j < 8; ++j) {
    const uint8_t *blk = p + 34 * j;
    s->sc[j] = 1;
    s->mn[j] = 0;
    s->dj[j] = oracle_half_to_double(rd16(blk));
    s->mj[j] = 0.0;
    for (int i = 0; i < 32; ++i) s->code[32 * j + i] = (int8_t)blk[2 + i];
  }
}

/* For the superblock formats the per-sub-block multipliers are d*sc_j and
 * dmin*m_j (each exact in fp64: 11 + 8 significant bits). */
static void fill_multipliers(oracle_sb *s) {
  for (int j = 0; j < s->nsub; ++j) {
    s->dj[j] = s->d * (double)s->sc[j];
    s->mj[j] = s->dmin * (double)s->mn[j];
  }
}

static int decode_sb(int type, const uint8_t *p, oracle_sb *s) {
  switch (type) {
    case OR_Q4_K: decode_q4_k(p, s); fill_multipliers(s); return 0;
    case OR_Q6_K: decode_q6_k(p, s); fill_multipliers(s); return 0;
    case OR_IQ4_XS: decode_iq4_xs(p, s); fill_multipliers(s); return 0;
    case OR_Q4_0: decode_q4_0(p, s); return 0;
    case OR_Q8_0: decode_q8_0(p, s); return 0;
    default: return -1;
  }
}

static int check_args(int type, int64_t N, int64_t K, int64_t M) {
  if (block_bytes(type) == 0) return -1;
  if (N < 1 || M < 1 || K < OR_QK || K % OR_QK != 0) return -1;
  return 0;
}

/* Exact dequantization w[n][k] (fp64; every value is exact, see header). */
int oracle_dequant(const uint8_t *W, int type, int64_t N, int64_t K, double *w) {
  if (check_args(type, N, K, 1)) return -1;
  int bb = block_bytes(type);
  int64_t nsb = K / OR_QK;
  oracle_sb s;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nsb; ++b) {
      decode_sb(type, W + (n * nsb + b) * bb, &s);
      for (int e = 0; e < OR_QK; ++e) {
        int j = e / s.sublen;
        w[n * K + b * OR_QK + e] = s.dj[j] * (double)s.code[e] - s.mj[j];
      }
    }
  return 0;
}

/* Integer sub-block sums I[m][n][k/S] = sum over the sub-block of
 * code_w * q_x (S = 16 for Q6_K, 32 for every other format).  These are the
 * exact int32 block dots of the Kestrel page, section 5. */
int oracle_isums(const uint8_t *W, int type, int64_t N, int64_t K,
                 const uint8_t *xq, int64_t M, int64_t *isums) {
  if (check_args(type, N, K, M)) return -1;
  int bb = block_bytes(type);
  int64_t nsb = K / OR_QK, nq8 = K / OR_Q8_BLOCK;
  oracle_sb s0;
  decode_sb(type, W, &s0); /* for sublen */
  int64_t nsubrow = K / s0.sublen;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t b = 0; b < nsb; ++b) {
      oracle_sb s;
      decode_sb(type, W + (n * nsb + b) * bb, &s);
      for (int64_t m = 0; m < M; ++m)
        for (int j = 0; j < s.nsub; ++j) {
          int64_t acc = 0;
          for (int i = 0; i < s.sublen; ++i) {
            int64_t k = b * OR_QK + j * s.sublen + i;
            const uint8_t *blk = xq + (m * nq8 + k / OR_Q8_BLOCK) * OR_Q8_BYTES;
            acc += (int64_t)s.code[j * s.sublen + i] * (int8_t)blk[4 + k % OR_Q8_BLOCK];
          }
          isums[(m * N + n) * nsubrow + b * s.nsub + j] = acc;
        }
    }
  return 0;
}

/* The matmul: y[m][n] = sum over superblocks b and sub-blocks j of
 *   Q4_K  : d*sc_j*D*I_j - dmin*m_j*S
 *   Q6_K  : d*sc_t*D*I_t
 *   IQ4_XS: d*(ls_j-32)*D*I_j
 * where D, S belong to the Q8_1 block that holds the sub-block's activations.
 * Outputs: y64 (fp64 sum in K order), absum = sum of |terms| (the scale of the
 * rounding error, used by tolerance checks) and y32 = y64 rounded to fp32.
 * Any of the three output pointers may be NULL. */
int oracle_qmatmul(const uint8_t *W, int type, int64_t N, int64_t K,
                   const uint8_t *xq, int64_t M, double *y64, double *absum,
                   float *y32) {
  if (check_args(type, N, K, M)) return -1;
  int bb = block_bytes(type);
  int64_t nsb = K / OR_QK, nq8 = K / OR_Q8_BLOCK;
#pragma omp parallel for collapse(2) schedule(dynamic, 16)
  for (int64_t m = 0; m < M; ++m)
    for (int64_t n = 0; n < N; ++n) {
      double acc = 0.0, aabs = 0.0;
      for (int64_t b = 0; b < nsb; ++b) {
        oracle_sb s;
        decode_sb(type, W + (n * nsb + b) * bb, &s);
        for (int j = 0; j < s.nsub; ++j) {
          int64_t k0 = b * OR_QK + (int64_t)j * s.sublen;
          const uint8_t *blk = xq + (m * nq8 + k0 / OR_Q8_BLOCK) * OR_Q8_BYTES;
          double D = oracle_half_to_double(rd16(blk));
          double S = oracle_half_to_double(rd16(blk + 2));
          int64_t I = 0;
          for (int i = 0; i < s.sublen; ++i)
            I += (int64_t)s.code[j * s.sublen + i] *
                 (int8_t)blk[4 + (k0 + i) % OR_Q8_BLOCK];
          double term = (s.dj[j] * D) * (double)I; /* exact */
          acc += term;
          aabs += fabs(term);
          if (s.mn[j] != 0) {
            double mterm = s.mj[j] * S; /* exact */
            acc -= mterm;
            aabs += fabs(mterm);
          }
        }
      }
      if (y64) y64[m * N + n] = acc;
      if (absum) absum[m * N + n] = aabs;
      if (y32) y32[m * N + n] = (float)acc;
    }
  return 0;
}

/* Same matmul restricted to a list of output rows (n indices), for sampled
 * checks at full size: y64[m][r] is output (m, rows[r]). */
int oracle_qmatmul_rows(const uint8_t *W, int type, int64_t N, int64_t K,
                        const uint8_t *xq, int64_t M, const int64_t *rows,
                        int64_t nrows, double *y64, double *absum) {
  if (check_args(type, N, K, M) || nrows < 0) return -1;
  int64_t row_bytes = (K / OR_QK) * block_bytes(type);
  for (int64_t r = 0; r < nrows; ++r) {
    if (rows[r] < 0 || rows[r] >= N) return -1;
  }
  int fail = 0;
#pragma omp parallel
  {
    double *t64 = (double *)malloc(sizeof(double) * (size_t)M);
    double *tab = (double *)malloc(sizeof(double) * (size_t)M);
    if (!t64 || !tab) {
#pragma omp atomic write
      fail = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
      if (!t64 || !tab) continue;
      /* one output row: the single-row matmul above, run by this thread */
      oracle_qmatmul(W + rows[r] * row_bytes, type, 1, K, xq, M, t64, tab, NULL);
      for (int64_t m = 0; m < M; ++m) {
        if (y64) y64[m * nrows + r] = t64[m];
        if (absum) absum[m * nrows + r] = tab[m];
      }
    }
    free(t64);
    free(tab);
  }
  return fail ? -2 : 0;
}

/* ------------------------------------------------ int4-KV decode attention */

/* One decode step of attention over a 4-bit KV cache (xLLM v0.7 log, section
 * C.3: the long-context path runs paged attention with int4 K/V dot products
 * over the whole context; Kestrel_VLLM #18, the online-softmax decode kernel:
 * the query is quantized to int8, Q.K is an int32 dot, then softmax and a
 * sequential P.V sum).  The pages do not print the int4 KV layout.  Readings:
 *   - K and V rows of D elements are D/32 Q4_0 blocks (the pages' simplest
 *     4-bit block: fp16 d, 16 bytes of nibbles, element i low nibble of byte
 *     i, element 16 + i high nibble, value d * (q - 8));
 *   - the cache is [Hkv][T][D/32 blocks]; query head h reads KV head
 *     h / (Hq / Hkv) (grouped-query attention, consecutive heads share);
 *   - the query is Q8_1 blocks [Hq][D/32] (the activation quantizer above);
 *   - score s_t = scale * sum_b dK_b * D_b * I_b, I_b the exact integer dot
 *     of block b's codes (q - 8) with the query's int8 codes; no mask.
 * Then, per query head, in fp64 and in token order:
 *   m = max_t s_t;  p_t = exp(s_t - m);  l = sum_t p_t;
 *   out[d] = (sum_t p_t * v_t[d]) / l,  v_t[d] = dV * (q - 8).
 * scores (optional) receives s [Hq][T]; out is fp64 [Hq][D].  Returns 0, or
 * -1 for bad arguments (T < 1, D % 32, Hq % Hkv). */
int oracle_attn_decode_kv4(const uint8_t *q_q8, int64_t Hq, const uint8_t *Kc,
                           const uint8_t *Vc, int64_t Hkv, int64_t T, int64_t D,
                           double scale, double *out, double *scores) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv || T < 1 || D < 32 || D % 32) return -1;
  const int64_t nb = D / 32, row = nb * 18, G = Hq / Hkv;
  double *s = (double *)malloc(sizeof(double) * (size_t)T);
  if (!s) return -2;
  for (int64_t h = 0; h < Hq; ++h) {
    const int64_t g = h / G;
    const uint8_t *qh = q_q8 + h * nb * OR_Q8_BYTES;
    const uint8_t *Kh = Kc + g * T * row, *Vh = Vc + g * T * row;
    for (int64_t t = 0; t < T; ++t) {
      double acc = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *kb = Kh + t * row + b * 18, *qb = qh + b * OR_Q8_BYTES;
        int64_t I = 0;
        for (int i = 0; i < 16; ++i) {
          I += (int64_t)((kb[2 + i] & 15) - 8) * (int8_t)qb[4 + i];
          I += (int64_t)((kb[2 + i] >> 4) - 8) * (int8_t)qb[4 + 16 + i];
        }
        acc += oracle_half_to_double(rd16(kb)) * oracle_half_to_double(rd16(qb)) * (double)I;
      }
      s[t] = scale * acc;
      if (scores) scores[h * T + t] = s[t];
    }
    double m = s[0];
    for (int64_t t = 1; t < T; ++t)
      if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      s[t] = exp(s[t] - m);
      l += s[t];
    }
    for (int64_t d = 0; d < D; ++d) {
      const int64_t b = d / 32, i = d % 32;
      double o = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const uint8_t *vb = Vh + t * row + b * 18;
        const int code = i < 16 ? (vb[2 + i] & 15) : (vb[2 + i - 16] >> 4);
        o += s[t] * (oracle_half_to_double(rd16(vb)) * (double)(code - 8));
      }
      out[h * D + d] = o / l;
    }
  }
  free(s);
  return 0;
}
