// attn_kv4.hip -- one decode step of attention over a 4-bit KV cache: the
// long-context path of the xLLM v0.7 log (section C.3: paged attention with
// int4 K/V dot products over the whole context, a working set that misses L2,
// so every step streams the cache from HBM), with the integer Q.K of the
// Kestrel #18 decode kernel (int8 query, int32 dot, then softmax and P.V).
//
// Layout: K and V rows of D = 128 elements are four Q4_0 blocks (fp16 d and
// 16 bytes of nibbles; element i is the low nibble of byte i, element 16 + i
// the high nibble; value d * (q - 8)), 72 bytes a row, cache [Hkv][T][row];
// the query is Q8_1 blocks [Hq][4]; query head h reads KV head h / G, G =
// Hq / Hkv.
//
// Two kernels, split over the context (flash-decoding):
//   attn_kv4_partial  one workgroup per (256-token chunk, KV head) serves the
//                     G query heads of that KV head, so each K and V byte is
//                     read from HBM once per step.  The chunk's K and V rows
//                     are staged in LDS by coalesced loads, all issued before
//                     the first wait.  Scores: exact int32 dots
//                     (v_dot4_i32_i8 on the nibbles, minus 8 * the query
//                     block's code sum), the scale products and the four
//                     blocks summed in fp64 (every product exact) and rounded
//                     once to fp32.  Softmax over the chunk in fp32 (max,
//                     expf, fixed-order sums), then P.V from the V rows staged
//                     in LDS; writes the chunk's max m, sum l and unnormalised
//                     output o[128] per head to the workspace.
//   attn_kv4_combine  per (head, 32 outputs): M = max m_c, L = sum l_c
//                     e^(m_c - M), out = sum o_c e^(m_c - M) / L, the chunks
//                     in 16 residues joined in a fixed order.
#include "qdot_common.hpp"

namespace qdot {

constexpr int AT_D = 128;              // head dimension
constexpr int AT_NB = AT_D / 32;       // Q4_0 blocks per row
constexpr int AT_ROW = AT_NB * 18;     // bytes per K or V row
constexpr int AT_CH = 256;             // tokens per chunk (one per thread)
constexpr int AT_THREADS = 256;
constexpr int AT_WAVES = AT_THREADS / 64;
static_assert(AT_ROW % 8 == 0, "rows are staged in 8-byte pieces");

// 32 bits of a row held as 18 little-endian dwords, from byte offset off
// (known at compile time once unrolled).
__device__ __forceinline__ uint32_t row_u32(const uint32_t* kw, int off) {
  const int k = off >> 2, r = off & 3;
  return r == 0 ? kw[k] : __builtin_amdgcn_alignbyte(kw[k + 1], kw[k], r);
}

template <int G>
__global__ __launch_bounds__(AT_THREADS) void attn_kv4_partial_kernel(
    const uint8_t* __restrict__ q_q8, const uint8_t* __restrict__ Kc, const uint8_t* __restrict__ Vc,
    int T, int nchunks, float scale, float* __restrict__ ws_o, float* __restrict__ ws_m,
    float* __restrict__ ws_l) {
  __shared__ uint32_t q_codes[G][AT_NB][8];     // the query's int8 codes, 4 per dword
  __shared__ double q_d[G][AT_NB];              // the query blocks' D
  __shared__ int q_sum[G][AT_NB];               // sum of each query block's codes
  __shared__ float w_red[AT_WAVES][G];          // per-wave max
  __shared__ float w_sum[AT_WAVES][G];          // per-wave sum
  __shared__ __attribute__((aligned(16))) u32x2 v_s[AT_CH * AT_ROW / 8];  // the chunk's V rows
  // the chunk's K rows until the scores are formed; then the softmax
  // numerators p_s[G][AT_CH] during P.V, and after it the per-wave P.V
  // partials o_red[AT_WAVES][G][AT_D]
  __shared__ __attribute__((aligned(16))) u32x2 k_s[AT_CH * AT_ROW / 8];
  static_assert(AT_WAVES * G * AT_D * sizeof(float) <= sizeof(k_s), "P.V partials fit the K stage");
  static_assert(G * AT_CH * sizeof(float) <= sizeof(k_s), "numerators fit the K stage");
  float (*p_s)[AT_CH] = reinterpret_cast<float (*)[AT_CH]>(k_s);
  float (*o_red)[G][AT_D] = reinterpret_cast<float (*)[G][AT_D]>(k_s);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int t0 = c * AT_CH;
  const int ntok = min(AT_CH, T - t0);
  const size_t row0 = (size_t)kvh * T + t0;

  // Every global load of the chunk goes out first, coalesced: this
  // thread's nine 8-byte pieces of the chunk's K rows and nine of its V rows
  // (indices clamped into the chunk, stored to LDS only when in range), so
  // all of them are in flight together.
  constexpr int VP = AT_CH * AT_ROW / 8 / AT_THREADS;  // pieces per thread and cache
  u32x2 kreg[VP], vreg[VP];
  const int npieces = ntok * (AT_ROW / 8);
  {
    const u32x2* ksrc = reinterpret_cast<const u32x2*>(Kc + row0 * AT_ROW);
    const u32x2* vsrc = reinterpret_cast<const u32x2*>(Vc + row0 * AT_ROW);
#pragma unroll
    for (int k = 0; k < VP; ++k) kreg[k] = ksrc[min(tid + k * AT_THREADS, npieces - 1)];
#pragma unroll
    for (int k = 0; k < VP; ++k) vreg[k] = vsrc[min(tid + k * AT_THREADS, npieces - 1)];
  }

  // query blocks of this KV head's G query heads
  if (tid < G * AT_NB) {
    const int g = tid / AT_NB, b = tid % AT_NB;
    const uint8_t* qb = q_q8 + ((size_t)(kvh * G + g) * AT_NB + b) * Q8_BYTES;
    q_d[g][b] = (double)h2f(ld4(qb));
    int s = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t w = ld4(qb + 4 + 4 * k);
      q_codes[g][b][k] = w;
      s += (int)(int8_t)(w & 255) + (int)(int8_t)((w >> 8) & 255) + (int)(int8_t)((w >> 16) & 255) +
           (int)(int8_t)(w >> 24);
    }
    q_sum[g][b] = s;
  }
  // stage the chunk's K and V rows
#pragma unroll
  for (int k = 0; k < VP; ++k)
    if (tid + k * AT_THREADS < npieces) {
      k_s[tid + k * AT_THREADS] = kreg[k];
      v_s[tid + k * AT_THREADS] = vreg[k];
    }
  __syncthreads();

  // scores: token t0 + tid
  float s_own[G];
  if (tid < ntok) {
    uint32_t kw[AT_ROW / 4];
#pragma unroll
    for (int k = 0; k < AT_ROW / 8; ++k) {
      const u32x2 v = k_s[tid * (AT_ROW / 8) + k];
      kw[2 * k] = v.x;
      kw[2 * k + 1] = v.y;
    }
    double acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
    for (int b = 0; b < AT_NB; ++b) {
      const double dk = (double)h2f(row_u32(kw, 18 * b) & 0xFFFFu);
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = row_u32(kw, 18 * b + 2 + 4 * k);
        lo[k] = w & 0x0F0F0F0Fu;          // elements 4k .. 4k+3
        hi[k] = (w >> 4) & 0x0F0F0F0Fu;   // elements 16+4k .. 16+4k+3
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        int I = -8 * q_sum[g][b];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          I = dot4(lo[k], q_codes[g][b][k], I);
          I = dot4(hi[k], q_codes[g][b][4 + k], I);
        }
        acc[g] += (dk * q_d[g][b]) * (double)I;   // exact product, fp64 sum in block order
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) s_own[g] = (float)((double)scale * acc[g]);
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) s_own[g] = -__builtin_inff();
  }

  // chunk max per head
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = s_own[g];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) w_red[wave][g] = m;
  }
  __syncthreads();  // also: every K row has been read, so k_s now takes p_s
  float mx[G];
#pragma unroll
  for (int g = 0; g < G; ++g) mx[g] = fmaxf(fmaxf(w_red[0][g], w_red[1][g]), fmaxf(w_red[2][g], w_red[3][g]));
  // numerators and their sum (butterfly in a fixed order, then the waves in order)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float p = tid < ntok ? expf(s_own[g] - mx[g]) : 0.0f;
    p_s[g][tid] = p;
    float l = p;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) w_sum[wave][g] = l;
  }
  __syncthreads();

  // P.V: wave w takes tokens 64w .. 64w+63 of the chunk, half-wave hw = l/32
  // the 32 tokens 64w + 32hw ..; lane l owns elements 32b + 2i, 32b + 2i + 1
  // (low nibbles of code bytes 2i, 2i+1 of block b) and the same + 16 (high
  // nibbles), b = (l%32)/8, i = l%8: one fp16 scale and one 16-bit code read
  // per token for four values
  {
    const int hw = lane >> 5, b = (lane & 31) >> 3, i2 = 2 * (lane & 7);
    float acc[4][G];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int g = 0; g < G; ++g) acc[e][g] = 0.0f;
    const uint8_t* vb = reinterpret_cast<const uint8_t*>(v_s);
    const int tbeg = 64 * wave + 32 * hw;
    const int tend = min(ntok, tbeg + 32);
    // the four values of token t for this lane, exact: d * q - 8 * d = d * (q - 8)
    // (fp16 d times a 4-bit code is exact in fp32, and so is the fma)
    auto vquad = [&](int t, float (&v)[4]) {
      const uint8_t* blk = vb + t * AT_ROW + 18 * b;
      const float dv = h2f(*reinterpret_cast<const uint16_t*>(blk));
      const uint32_t code = *reinterpret_cast<const uint16_t*>(blk + 2 + i2);
      const uint32_t lo = code & 0x0F0Fu, hi = (code >> 4) & 0x0F0Fu;
      const float m8 = -8.0f * dv;
      v[0] = fmaf(dv, (float)(lo & 0xFFu), m8);   // element 32b + i2
      v[1] = fmaf(dv, (float)(lo >> 8), m8);      // 32b + i2 + 1
      v[2] = fmaf(dv, (float)(hi & 0xFFu), m8);   // 32b + 16 + i2
      v[3] = fmaf(dv, (float)(hi >> 8), m8);      // 32b + 16 + i2 + 1
    };
    // four tokens a step (p of the four tokens in one 16-byte read), the sums
    // in token order
    int t = tbeg;
    for (; t + 4 <= tend; t += 4) {
      float v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) vquad(t + u, v[u]);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float4 p4 = *reinterpret_cast<const float4*>(&p_s[g][t]);
        const float pu[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e][g] = fmaf(pu[u], v[u][e], acc[e][g]);
      }
    }
    for (; t < tend; ++t) {
      float v[4];
      vquad(t, v);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = p_s[g][t];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e][g] = fmaf(p, v[e], acc[e][g]);
      }
    }
    // the two half-waves' partials: first half + second half
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float other = __shfl_xor(acc[e][g], 32, 64);
        acc[e][g] = hw == 0 ? acc[e][g] + other : other + acc[e][g];
      }
    __syncthreads();  // every wave is done with p_s before o_red overwrites it
    if (hw == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        o_red[wave][g][32 * b + i2] = acc[0][g];
        o_red[wave][g][32 * b + i2 + 1] = acc[1][g];
        o_red[wave][g][32 * b + 16 + i2] = acc[2][g];
        o_red[wave][g][32 * b + 16 + i2 + 1] = acc[3][g];
      }
    }
  }
  __syncthreads();
  for (int o = tid; o < G * AT_D; o += AT_THREADS) {
    const int g = o / AT_D, d = o % AT_D;
    const float v = ((o_red[0][g][d] + o_red[1][g][d]) + o_red[2][g][d]) + o_red[3][g][d];
    ws_o[((size_t)(kvh * G + g) * nchunks + c) * AT_D + d] = v;
  }
  if (tid < G) {
    const size_t i = (size_t)(kvh * G + tid) * nchunks + c;
    ws_m[i] = mx[tid];
    ws_l[i] = ((w_sum[0][tid] + w_sum[1][tid]) + w_sum[2][tid]) + w_sum[3][tid];
  }
}

// One workgroup per (query head, 32 output elements): 16 x 32 threads,
// thread (k, e) sums element e of the slice over the partials c = k
// (mod 16); the sixteen partial sums, the max and the denominator are joined
// in a fixed order, so the result depends on the number of partials only.
constexpr int AC_SPLIT = 16, AC_COLS = 32;
__global__ __launch_bounds__(AC_SPLIT * AC_COLS) void attn_kv4_combine_kernel(const float* __restrict__ ws_o,
                                                                              const float* __restrict__ ws_m,
                                                                              const float* __restrict__ ws_l,
                                                                              int nparts, float* __restrict__ out) {
  constexpr int NT = AC_SPLIT * AC_COLS, NW = NT / 64;
  __shared__ float red_m[NW];
  __shared__ float red_l[NW];
  __shared__ float o_s[AC_SPLIT][AC_COLS];
  const int h = blockIdx.x, d0 = blockIdx.y * AC_COLS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = tid / AC_COLS, e = tid % AC_COLS;
  const float* m = ws_m + (size_t)h * nparts;
  const float* l = ws_l + (size_t)h * nparts;
  const float* o = ws_o + (size_t)h * nparts * AT_D + d0 + e;
  float mx = -__builtin_inff();
  for (int c = tid; c < nparts; c += NT) mx = fmaxf(mx, m[c]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s, 64));
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  float M = red_m[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red_m[w]);
  // denominator: partial c by thread c (mod 512), then the waves in order
  float Lp = 0.0f;
  for (int c = tid; c < nparts; c += NT) Lp = fmaf(l[c], expf(m[c] - M), Lp);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) Lp += __shfl_xor(Lp, s, 64);
  if (lane == 0) red_l[wave] = Lp;
  float O = 0.0f;
#pragma unroll 4
  for (int c = k; c < nparts; c += AC_SPLIT) O = fmaf(o[(size_t)c * AT_D], expf(m[c] - M), O);
  o_s[k][e] = O;
  __syncthreads();
  if (k == 0) {
    float L = red_l[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) L += red_l[w];
    float v = o_s[0][e];
#pragma unroll
    for (int i = 1; i < AC_SPLIT; ++i) v += o_s[i][e];
    out[(size_t)h * AT_D + d0 + e] = v / L;
  }
}

size_t attn_kv4_workspace_bytes(int64_t Hq, int64_t T) {
  const int64_t nchunks = (T + AT_CH - 1) / AT_CH;
  return (size_t)Hq * (size_t)nchunks * (AT_D + 2) * sizeof(float);
}

template <int G>
static int launch_partial(const uint8_t* q, const uint8_t* K, const uint8_t* V, int Hkv, int T,
                          int nchunks, float scale, float* wo, float* wm, float* wl, hipStream_t s) {
  hipLaunchKernelGGL((attn_kv4_partial_kernel<G>), dim3(nchunks, Hkv), dim3(AT_THREADS), 0, s, q, K, V, T,
                     nchunks, scale, wo, wm, wl);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Arguments are validated by the caller (api.cpp): D = 128, 1 <= G <= 8,
// T >= 1, workspace of attn_kv4_workspace_bytes(Hq, T) bytes.
int launch_attn_kv4(const void* q_q8, int Hq, const void* Kc, const void* Vc, int Hkv, int T, float scale,
                    float* out, void* workspace, hipStream_t s) {
  const int G = Hq / Hkv;
  const int nchunks = (T + AT_CH - 1) / AT_CH;
  float* wo = static_cast<float*>(workspace);
  float* wm = wo + (size_t)Hq * nchunks * AT_D;
  float* wl = wm + (size_t)Hq * nchunks;
  const uint8_t* q = static_cast<const uint8_t*>(q_q8);
  const uint8_t* K = static_cast<const uint8_t*>(Kc);
  const uint8_t* V = static_cast<const uint8_t*>(Vc);
  int rc;
  switch (G) {
    case 1: rc = launch_partial<1>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 2: rc = launch_partial<2>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 3: rc = launch_partial<3>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 4: rc = launch_partial<4>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 5: rc = launch_partial<5>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 6: rc = launch_partial<6>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 7: rc = launch_partial<7>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    case 8: rc = launch_partial<8>(q, K, V, Hkv, T, nchunks, scale, wo, wm, wl, s); break;
    default: return -2;
  }
  if (rc) return rc;
  hipLaunchKernelGGL(attn_kv4_combine_kernel, dim3(Hq, AT_D / AC_COLS), dim3(AC_SPLIT * AC_COLS), 0, s, wo, wm,
                     wl, nchunks, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace qdot
