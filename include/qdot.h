/*
 * qdot.h -- C ABI of the integer-dot block-quantized matmul for AMD MI355X
 * (gfx950).  Library: libqdot.so.
 *
 * The operation.  Decode in GGUF-quantized LLM inference multiplies raw
 * block-quantized weights (Q4_K, Q6_K, IQ4_XS superblocks of 256 weights;
 * Q4_0 and Q8_0 blocks of 32, taken eight at a time)
 * against activations quantized to Q8_1 blocks of 32, using integer dot
 * products on the raw quantized values, and only then produces fp32; the
 * weights are never dequantized to fp32 (xLLM v0.7 dev log,
 * developer.cloud.tencent.com.cn/article/2739032, section 1 "background" and
 * section B1.3).  Each activation quantization is shared by every row of the
 * batch (same page, section C, the shared d_xn_q8 buffer).  Inside each block
 * the dot is an exact int32 sum; the scales are applied afterwards (Kestrel
 * page, wsisp.com posts/117433, section 5).
 *
 * Formats (byte layouts; the pages name the formats, the layouts are the plain
 * GGUF reading):
 *   Q8_1   36 B per 32 activations: fp16 d, fp16 s, int8 q[32].
 *   Q4_K  144 B per 256 weights: fp16 d, fp16 dmin, 12 B of 6-bit scales and
 *         mins for 8 sub-blocks of 32, 128 B of 4-bit codes;
 *         w = d*sc*q - dmin*m.
 *   Q6_K  210 B per 256 weights: 128 B low 4 bits, 64 B high 2 bits, 16 int8
 *         sub-scales (sub-blocks of 16), fp16 d; w = d*sc*(q-32).
 *   IQ4_XS 136 B per 256 weights: fp16 d, u16 scales_h, 4 B scales_l (eight
 *         6-bit scales ls), 128 B of 4-bit codebook indices; each 32-element
 *         sub-block has low nibbles = elements 0-15 and high nibbles = 16-31
 *         (V100TPS log, agent-report.daedalus.work, 2026-08-12 "batch kernel
 *         locked to Q4_0"); w = d*(ls-32)*codebook[idx].  The 16-entry
 *         codebook is a placeholder (the pages do not print kvalues_iq4nl):
 *         round_half_away(-127 + 240*(i/15)^1.4), i = 0..15.
 *   Q4_0   18 B per 32 weights: fp16 d, 16 B of 4-bit codes, low nibbles =
 *         elements 0-15, high nibbles = 16-31 (V100TPS log, same entry);
 *         w = d*(q-8).  Eight blocks (144 B) form one 256-weight group.
 *   Q8_0   34 B per 32 weights: fp16 d, int8 q[32] (the xLLM page's 34-byte
 *         block, Phase B3/B4); w = d*q.  Eight blocks (272 B) form one
 *         256-weight group; blocks sit at 2-byte alignment.
 *
 * Layouts.  Every buffer is contiguous and row-major: x is fp32 [M][K];
 * x_q8 is [M][K/32] Q8_1 blocks; W is [N][K/256] superblocks (GGUF row
 * order, row n at W + n*row_bytes, so a row subset is W + n0*row_bytes with a
 * smaller N); y is fp32 [M][N].
 *
 * Ownership and threading.  The caller owns and allocates every buffer;
 * device pointers must be device memory of the current HIP device.  The
 * library never allocates, frees or synchronizes, keeps no mutable global
 * state (one exception: qdot_attn_decode_kv4_noalloc's static device
 * workspace and the per-device address it caches), and enqueues its kernels
 * on the caller's stream (0 = the null stream).  Calls are asynchronous and
 * thread-safe (qdot_attn_decode_kv4_noalloc: see its limits).
 *
 * Errors.  Arguments are validated before any HIP call; on failure nothing is
 * launched and a negative status is returned:
 *   QDOT_E_ARG   null pointer, M < 1, N < 1, K < 256 or K % 256 != 0 (K % 32
 *                != 0 for the quantizer), unknown type, or a size overflow;
 *   QDOT_E_ALIGN x, x_q8, y or isums not 4-byte aligned (W may sit at any
 *                byte address: the kernels read it with unaligned vector
 *                loads, as Q6_K superblocks of 210 bytes require);
 *   QDOT_E_HIP   the launch failed (hipGetLastError after the launch).
 * There is no fallback path and no environment variable.  Inputs must be
 * finite and each Q8_1 block's fp16 d and s finite; otherwise results are
 * undefined (but every launch stays in bounds).
 */
#ifndef QDOT_H
#define QDOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QDOT_Q4_K = 1, QDOT_Q6_K = 2, QDOT_IQ4_XS = 3, QDOT_Q4_0 = 4, QDOT_Q8_0 = 5
} qdot_type;

enum { QDOT_OK = 0, QDOT_E_ARG = -1, QDOT_E_ALIGN = -2, QDOT_E_HIP = -3 };

/* Bytes per 256 weights: 144 (Q4_K), 210 (Q6_K), 136 (IQ4_XS), 144 (Q4_0,
 * eight blocks), 272 (Q8_0, eight blocks); 0 for an unknown type. */
size_t qdot_block_bytes(int type);

/* Bytes of an N x K weight matrix: N * (K/256) * qdot_block_bytes(type);
 * 0 if the arguments are invalid. */
size_t qdot_weight_bytes(int type, int64_t N, int64_t K);

/* Bytes of M x K activations in Q8_1: M * (K/32) * 36; 0 if invalid. */
size_t qdot_q8_1_bytes(int64_t M, int64_t K);

/* Number of int32 sub-block sums written by qdot_qmatmul_dump_isums:
 * M * N * (K/S), S = 16 (Q6_K) or 32 (every other type); 0 if invalid. */
size_t qdot_isum_count(int type, int64_t N, int64_t K, int64_t M);

/* Quantize fp32 activations x [M][K] (device) to Q8_1 blocks x_q8 (device,
 * qdot_q8_1_bytes(M, K) bytes).  Per block of 32: amax = max|x_i|;
 * d32 = amax/127 (IEEE fp32 division); q_i = roundf(x_i/d32) (fp32 division,
 * ties away from zero) clamped to [-127, 127], all zero when amax == 0;
 * stored d = fp16(d32), stored s = fp16(d * sum q_i), both round to nearest
 * even.  The pages launch this quantizer once ahead of the matmul and share
 * it across the batch (V100TPS log, 2026-08-12, on ggml_mul_mat_a8; xLLM
 * page, section C).  K % 32 == 0 is required. */
int qdot_quantize_q8_1(const float *x, int64_t M, int64_t K, void *x_q8,
                       void *stream);

/* y [M][N] = x_q8 [M][K] (Q8_1) times W^T, W = [N][K] raw superblocks of
 * `type`.  Per output: sum over superblocks and sub-blocks of
 *   Q4_K   d*sc*D*I - dmin*m*S
 *   Q6_K   d*sc*D*I            (sub-blocks of 16)
 *   IQ4_XS d*(ls-32)*D*I
 *   Q4_0, Q8_0  d*D*I  (d the block's own scale; Q4_0 codes are q-8)
 * where I is the exact integer dot of the sub-block's weight codes with the
 * int8 activations and D, S are the activation block's fp16 d and s.  Every
 * scale product is exact and accumulated in fp64 (in the prefill kernel the
 * Q4_K min terms on the fp64 matrix cores); y is rounded once to fp32.
 * M <= 8 runs the decode kernel (v_dot4_i32_i8, M-row tile; for Q4_K at
 * M = 7, 8 and IQ4_XS at M = 5..8 the integer dots run on
 * v_mfma_i32_32x32x32_i8 instead, and for Q6_K at M = 7, 8 on
 * v_mfma_i32_16x16x32_i8, summed in the same order, so the rows are
 * bitwise those of the dot4 tile); Q4_K and IQ4_XS keep that MFMA decode
 * tile, with 16-row activation slots, up to M = 16.  Above the decode range
 * and up to M = 96 runs a mid-batch MFMA i8 kernel (16-row activation tiles,
 * K split eight ways); M > 96 the MFMA i8 prefill kernel (the mid-batch
 * kernel's upper end depends on the matrix: qdot_kernel_name_shape).  Within
 * each of these three ranges a row of y is bitwise the same whatever M it is
 * computed with; across them it may differ in the last fp32 bit (different
 * fp64 summation orders).  K % 256 == 0 is required.
 * The operation is the xLLM v0.7 log's integer-dot matmul on raw Q4_K / Q6_K
 * weights (section 1 "background"; section B2, the M-templated tile that
 * reads each weight once for all M rows), with the sub-block dot an exact
 * int32 sum and the scales applied after it (Kestrel_VLLM #18, section 5);
 * the IQ4_XS sub-block scale d*(ls-32) and its codebook lookup are the
 * V100TPS log's (2026-08-12 entries). */
int qdot_qmatmul(const void *W, int type, int64_t N, int64_t K,
                 const void *x_q8, int64_t M, float *y, void *stream);

/* Same as qdot_qmatmul (same kernel template, same y) and also writes every
 * integer sub-block sum I to isums [M][N][K/S] (int32, device,
 * qdot_isum_count elements): a debug dump for bit-exact checks against a CPU
 * reference, after the Kestrel_VLLM #18 page's practice of dumping the same
 * intermediate buffers on the CPU and the GPU side and diffing them to find
 * the first value that differs (section 3.4, the full-model dump harness). */
int qdot_qmatmul_dump_isums(const void *W, int type, int64_t N, int64_t K,
                            const void *x_q8, int64_t M, float *y,
                            int32_t *isums, void *stream);

/* Up to QDOT_MULTI_MAX weight matrices that read the same activation rows
 * (same K and M), e.g. the Q, K and V projections of an attention layer or
 * the gate and up projections of an FFN, in one launch: y[i] = W[i] x for
 * i < n, each exactly as qdot_qmatmul(W[i], types[i], N[i], K, x_q8, M, y[i])
 * computes it (bitwise the same y).  The pages fuse Q/K/V behind one shared
 * Q8_1 quantization (the IQ4_XS hidden-5120 model's QKV matrix; xLLM v0.7
 * log, section C.1, one activation quantization shared by every slot); this
 * call does the same without requiring the matrices to share a weight type.
 * W, types, N and y are host arrays of n entries; W[i] and y[i] are device
 * pointers with the alignment qdot_qmatmul requires.  For M <= 8 the decode
 * tiles of all matrices run in one launch (Q4_K with Q6_K, Q4_0 with Q8_0, or
 * a single type; other mixes take one launch per type), Q4_K and IQ4_XS
 * tiles on the MFMA units where that measured faster (K >= 4096); for M > 8
 * the matrices are launched one after another.  The saving is the fixed cost of
 * the launches replaced.  Errors as qdot_qmatmul; n outside 1..QDOT_MULTI_MAX
 * is E_ARG.  Every argument is checked before anything is launched. */
#define QDOT_MULTI_MAX 4
int qdot_qmatmul_multi(int n, const void *const *W, const int *types,
                       const int64_t *N, int64_t K, const void *x_q8,
                       int64_t M, float *const *y, void *stream);

/* The activation quantizer fused into the decode matmul: y = W x for fp32
 * activations x [M][K] (device, 4-byte aligned), computed as
 * qdot_qmatmul(W, type, N, K, quantize_q8_1(x), M) computes it -- bitwise
 * the same y -- in one launch instead of two.  Each wave of the decode
 * kernel quantizes the Q8_1 blocks of its own superblocks into LDS with the
 * standalone quantizer's code (readings as qdot_quantize_q8_1), so no Q8_1
 * buffer is written.  The pages launch quantize_q8_1 once ahead of the
 * matmul (V100TPS log, 2026-08-12, ggml_mul_mat_a8); on MI355X a launch costs
 * about as much as a small quantization, which is what the fusion saves.
 * Every workgroup quantizes the activations it reads, so the fused call pays
 * that work once per workgroup: it is meant for small M.  Runs the dot4
 * decode tile.  1 <= M <= QDOT_QUANTIZE_QMATMUL_MAX_M, else E_ARG; other
 * errors as qdot_qmatmul. */
#define QDOT_QUANTIZE_QMATMUL_MAX_M 8
int qdot_quantize_qmatmul(const void *W, int type, int64_t N, int64_t K,
                          const float *x, int64_t M, float *y, void *stream);

/* The same for up to QDOT_MULTI_MAX matrices that read the same activations
 * (qdot_qmatmul_multi's grouping, dot4 tiles): y[i] bitwise equal to
 * qdot_qmatmul(W[i], ..., quantize_q8_1(x), ...). */
int qdot_quantize_qmatmul_multi(int n, const void *const *W, const int *types,
                                const int64_t *N, int64_t K, const float *x,
                                int64_t M, float *const *y, void *stream);

/* RMSNorm fused with the Q8_1 quantizer: x_q8 = quantize_q8_1(RMSNorm(x) * w)
 * in one launch, for the producer of the Q/K/V and gate/up activations (the
 * xLLM v0.7 log, section C.1, quantizes the normalized input into one shared
 * buffer).  Per row of x [M][K] (fp32, device): ss = sum of x_k^2, r =
 * 1.0f / sqrtf(ss / K + eps), xn_k = (x_k * r) * w_k, all in fp32 with
 * correctly rounded division and square root as on the Kestrel_VLLM #18
 * page (section 3.6); ss is summed in that page's order (each group of 8
 * squares as lo_k = s_k + s_(k+4), (lo0 + lo1) + (lo2 + lo3), and the group
 * sums added left to right into one fp32 accumulator), so the output bytes
 * equal those of a plain serial CPU loop bit for bit.  xn
 * is then quantized exactly as qdot_quantize_q8_1 does.  w is fp32 [K]
 * (device); x_q8 receives qdot_q8_1_bytes(M, K) bytes.  32 <= K <=
 * QDOT_RMSNORM_MAX_K, K % 32 == 0, eps finite and >= 0, else E_ARG; x, w,
 * x_q8 4-byte aligned, else E_ALIGN. */
#define QDOT_RMSNORM_MAX_K 32768
int qdot_rmsnorm_quantize_q8_1(const float *x, const float *w, float eps,
                               int64_t M, int64_t K, void *x_q8, void *stream);

/* One decode step of attention over a 4-bit KV cache (the long-context path
 * of the xLLM v0.7 log, section C.3: paged attention with int4 K/V dot
 * products over the whole context, whose cache misses L2 and streams from
 * HBM every step; the integer Q.K of the Kestrel_VLLM #18 decode kernel, an
 * int8 query with an int32 dot product, then softmax and the P.V sum).
 * Layout (the pages print none; the reading): a K or V row of D elements is
 * D/32 Q4_0 blocks of 18 bytes (binary16 d, then 16 bytes; byte i holds
 * element i in its low nibble and element 16 + i in its high nibble; value
 * d * (q - 8)); Kc and Vc are [Hkv][T][row] (device, 8-byte aligned);
 * q_q8 is the query as Q8_1 blocks [Hq][D/32] (qdot_quantize_q8_1 of the
 * fp32 query [Hq][D]); query head h reads KV head h / (Hq / Hkv).
 *   s_t = scale * sum_b dK_b * D_b * I_b   (I_b the exact int32 dot of block
 *         b's codes q - 8 with the query's codes; the products exact, the
 *         blocks summed in fp64, rounded once to fp32)
 *   out[h][d] = sum_t e^(s_t - max s) v_t[d] / sum_t e^(s_t - max s)
 * in fp32 (expf; the context split in chunks of 256 tokens combined in
 * order), out fp32 [Hq][D] (device).  workspace: device scratch of at least
 * qdot_attn_kv4_workspace_bytes(Hq, T) bytes, 4-byte aligned, owned by the
 * caller and overwritten (calls on one workspace must not overlap).  No mask:
 * every one of the T tokens is attended.  Errors: QDOT_E_ARG for a null
 * pointer, D != QDOT_ATTN_HEAD_DIM, Hq % Hkv != 0, Hq / Hkv >
 * QDOT_ATTN_MAX_GROUP, Hq > QDOT_ATTN_MAX_HEADS, T outside 1..QDOT_ATTN_MAX_T,
 * a non-finite scale or a short workspace; QDOT_E_ALIGN for Kc, Vc not 8-byte
 * or q_q8, out, workspace not 4-byte aligned; QDOT_E_HIP if a launch fails. */
#define QDOT_ATTN_HEAD_DIM 128
#define QDOT_ATTN_MAX_GROUP 8
#define QDOT_ATTN_MAX_HEADS 4096
#define QDOT_ATTN_MAX_T (1 << 26)
int qdot_attn_decode_kv4(const void *q_q8, int64_t Hq, const void *Kc,
                         const void *Vc, int64_t Hkv, int64_t T, int64_t D,
                         float scale, float *out, void *workspace,
                         size_t workspace_bytes, void *stream);

/* qdot_attn_decode_kv4 for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and the same result, bit for bit, with the
 * workspace held in a static device array of QDOT_ATTN_NOALLOC_BYTES bytes
 * inside the library (each GPU the library runs on holds one copy until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current).  The call allocates and frees nothing.  Limit:
 * qdot_attn_kv4_workspace_bytes(Hq, T) <= QDOT_ATTN_NOALLOC_BYTES (e.g.
 * Hq = 32 up to T = 258,048 tokens), else QDOT_E_ARG.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents (nothing in
 * it has to start at zero): calls that overlap on one GPU (concurrent
 * streams, or host threads issuing calls that can run at the same time)
 * race and give wrong results; serialize them.  Other arguments, alignment
 * and errors as qdot_attn_decode_kv4; QDOT_E_HIP also if the array's device
 * address cannot be obtained. */
#define QDOT_ATTN_NOALLOC_BYTES (16 << 20)
int qdot_attn_decode_kv4_noalloc(const void *q_q8, int64_t Hq, const void *Kc,
                                 const void *Vc, int64_t Hkv, int64_t T,
                                 int64_t D, float scale, float *out,
                                 void *stream);

/* Bytes of one K or V row of D elements in qdot_attn_decode_kv4's cache
 * (D/32 blocks of 18 bytes); 0 unless D is a multiple of 32 in
 * 32..QDOT_ATTN_HEAD_DIM. */
size_t qdot_attn_kv4_row_bytes(int64_t D);

/* Workspace bytes qdot_attn_decode_kv4 needs for Hq query heads over T
 * tokens (per head and 256-token chunk: a max, a sum and D partial
 * outputs, fp32); 0 for Hq or T out of range. */
size_t qdot_attn_kv4_workspace_bytes(int64_t Hq, int64_t T);

/* Static text for a status code.  Failures are reported, never papered
 * over by a slower path: the xLLM v0.7 log's fail-fast rule (section A2.2,
 * a failed preload aborts loudly) and its explicit decode-mode contract
 * (section B1.2, a mismatch errors out instead of degrading). */
const char *qdot_status_str(int status);

/* Which kernel ran, so that a measurement names its arm (the V100TPS log
 * prints the live kernel path with every benchmark entry, e.g. the
 * 2026-08-12 batch-kernel entries).
 * Name of the kernel qdot_qmatmul runs for (type, M) on a matrix of the
 * default ranges (decode tile for M <= 8, and for M <= 16 with Q4_K and
 * IQ4_XS; M <= 96 mid-batch kernel; larger M prefill kernel), e.g.
 * "qmv_dot4<Q4_K,4>", "qmv_mfma<Q4_K,8>", "qmv_mfma<IQ4_XS,12>",
 * "qmm_skinny<Q4_K>" or "qmm_mfma<Q6_K>"; "invalid" for bad arguments.  Static
 * text.  Exact for the decode names and for IQ4_XS below N = 8192, Q4_0 and
 * Q8_0; qdot_kernel_name_shape is exact for every matrix. */
const char *qdot_kernel_name(int type, int64_t M);

/* Name of the kernel qdot_qmatmul runs for a type-`type` N x K matrix and M
 * activation rows; "invalid" if the dimensions would be rejected.  The
 * mid-batch kernel's range depends on the matrix: up to M = 32 for Q4_K and
 * 48 for IQ4_XS when N >= 8192 and K >= 4096; up to 256 for Q6_K with
 * N <= 2048 and 128 for other Q6_K; up to 128 for Q4_K with N <= 2048; else
 * up to 96.  Static text. */
const char *qdot_kernel_name_shape(int type, int64_t N, int64_t K, int64_t M);

/* Name of the tile matrix i of a qdot_qmatmul_multi call with these types,
 * row counts, K and M runs: for M <= 8 "qmv_mfma<Q4_K,M>" / "qmv_mfma<IQ4_XS,M>"
 * where the group takes the MFMA tile (a choice made per launch, so it can
 * differ from the matrix's own qdot_kernel_name), else "qmv_dot4<type,M>";
 * for M > 8 qdot_kernel_name_shape of the matrix.  "invalid" if the call would
 * be rejected or i is out of range.  Static text. */
const char *qdot_multi_kernel_name(int n, const int *types, const int64_t *N,
                                   int64_t K, int64_t M, int i);

/* Measurement reference, not part of the matmul path: reads `bytes` bytes
 * at src (device, 16-byte aligned, bytes a positive multiple of 16) once with
 * coalesced 16-byte loads and no arithmetic beyond an XOR fold, the plain
 * read-only rate the HBM-bound decode launches are compared with (the pages
 * judge a kernel by its bandwidth against what the memory delivers: xLLM
 * v0.7 log, section B2, the ncu DRAM-throughput table).  sink: one device
 * dword, written only when the fold hits a fixed improbable value.  Errors:
 * E_ARG for null pointers or a bad size, E_ALIGN, E_HIP. */
int qdot_stream_read(const void *src, int64_t bytes, uint32_t *sink,
                     void *stream);

/* Build identifier of the library (compile date and time).  Static text. */
const char *qdot_build_id(void);

#ifdef __cplusplus
}
#endif

#endif /* QDOT_H */
