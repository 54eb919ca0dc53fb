// api.cpp -- the C ABI of libqdot (declared in include/qdot.h): argument
// validation (before any HIP call), kernel selection and launch on the
// caller's stream.  No allocation, no synchronization, no mutable globals,
// no environment variables, no fallback path: the caller states M and the
// weight type, and a bad argument fails loudly (the xLLM v0.7 log, section
// B1.2, gives the reason: a silently degraded path cost a 100x cliff).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qdot.h"

namespace qdot {
int launch_quantize_q8_1(const float* x, int64_t M, int64_t K, void* xq, hipStream_t s);
int launch_rmsnorm_q8_1(const float* x, const float* w, float eps, int64_t M, int64_t K, void* xq,
                        hipStream_t s);
int launch_qmv(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s);
int launch_qmm(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s);
int launch_qmm_skinny(const void* W, int type, int N, int K, const void* xq, int M, float* y,
                      int32_t* isums, hipStream_t s);
int launch_qmv_multi(int n, const void* const* W, const int* types, const int* N, int K, const void* xq,
                     int M, float* const* y, bool xf, hipStream_t s);
int launch_qmv_x(const void* W, int type, int N, int K, const float* x, int M, float* y, hipStream_t s);
bool qmv_multi_uses_mfma(int n, const int* types, const int* N, int K, int M, int i);
int launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
}  // namespace qdot

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;  // kernels index N, K with int

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int sub_len(int type) { return type == QDOT_Q6_K ? 16 : 32; }

// Validates everything but pointers; 0 or a status.
int check_dims(int type, int64_t N, int64_t K, int64_t M) {
  if (qdot_block_bytes(type) == 0) return QDOT_E_ARG;
  if (N < 1 || M < 1 || K < 256 || K % 256 != 0) return QDOT_E_ARG;
  if (N > kMaxDim || K > kMaxDim || M > kMaxDim) return QDOT_E_ARG;
  // products that index memory must fit in 63 bits
  if ((double)N * (double)(K / 256) * (double)qdot_block_bytes(type) > 9.0e18) return QDOT_E_ARG;
  if ((double)M * (double)N * (double)(K / 16) > 9.0e18) return QDOT_E_ARG;
  return QDOT_OK;
}

// Mid-batch dispatch: 9 <= M <= mid_max_m(type, N, K) runs the mid-batch
// MFMA kernel (16 activation rows per tile, K split eight ways), larger M the
// prefill kernel (64 or 32 activation rows per tile).  Measured on MI355X at
// the Qwen3-8B shapes the mid-batch kernel beats running the decode kernel
// over 8-row chunks at every M from 9 to 32 (4096 x 4096, M = 16: 11.8 vs
// 15.8 us), and over a whole layer it is faster up to M = 96 (M = 96: 368 vs
// 415 us on the prefill kernel at M = 97).  Wide matrices are the exception,
// since the prefill kernel stays flat in M up to 64 rows: 12288 x 4096 Q4_K
// takes 39.7-40.9 us there at M = 40..64 against 47.8-59.6 on the mid-batch
// kernel, and 58.4 against 86.0 at M = 96; 17408 x 5120 IQ4_XS 80.6 against
// 94.3 at M = 56 (but 79.0 against 75.3 at M = 48).  Q6_K stays on the
// mid-batch kernel (down 4096 x 12288 at M = 97: 157 us prefill, 100 us
// mid-batch at 96).  Above M = 96 the mid-batch kernel still wins on Q6_K and
// on narrow Q4_K matrices, the prefill kernel's Q6_K drain and its few
// workgroups for N <= 2048 being slow: v (1024 x 4096 Q6_K) 17.4 / 26.0 us at
// M = 128 / 256 against 41.3 / 41.6; k (1024 x 4096 Q4_K) 13.3 against 22.4
// at 128, equal at 160; down (4096 x 12288 Q6_K) 129 against 162 at 128,
// equal at 160, 188 against 162 at 192.  For a given matrix the switch
// happens at one M, so its rows stay the same for every M on either side.
#ifndef QDOT_SKINNY_MAX_M
#define QDOT_SKINNY_MAX_M 96
#endif

int64_t mid_max_m(int type, int64_t N, int64_t K) {
  if (N >= 8192 && K >= 4096) {
    if (type == QDOT_Q4_K) return 32;
    if (type == QDOT_IQ4_XS) return 48;
  }
  if (type == QDOT_Q6_K) return N <= 2048 ? 256 : 128;
  if (type == QDOT_Q4_K && N <= 2048) return 128;
  return QDOT_SKINNY_MAX_M;
}

int run_qmatmul(const void* W, int type, int64_t N, int64_t K, const void* x_q8, int64_t M,
                float* y, int32_t* isums, void* stream, bool dump) {
  int st = check_dims(type, N, K, M);
  if (st) return st;
  if (!W || !x_q8 || !y || (dump && !isums)) return QDOT_E_ARG;
  if (!aligned4(x_q8) || !aligned4(y) || (dump && !aligned4(isums))) return QDOT_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int rc = 0;
  if (M <= 8 || (M <= 16 && (type == QDOT_Q4_K || type == QDOT_IQ4_XS))) {
    rc = qdot::launch_qmv(W, type, (int)N, (int)K, x_q8, (int)M, y, dump ? isums : nullptr, s);
  } else if (M <= mid_max_m(type, N, K)) {
    rc = qdot::launch_qmm_skinny(W, type, (int)N, (int)K, x_q8, (int)M, y, dump ? isums : nullptr, s);
  } else {
    rc = qdot::launch_qmm(W, type, (int)N, (int)K, x_q8, (int)M, y, dump ? isums : nullptr, s);
  }
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

}  // namespace

extern "C" {

size_t qdot_block_bytes(int type) {
  switch (type) {
    case QDOT_Q4_K: return 144;
    case QDOT_Q6_K: return 210;
    case QDOT_IQ4_XS: return 136;
    case QDOT_Q4_0: return 8 * 18;
    case QDOT_Q8_0: return 8 * 34;
    default: return 0;
  }
}

size_t qdot_weight_bytes(int type, int64_t N, int64_t K) {
  if (check_dims(type, N, K, 1)) return 0;
  return (size_t)N * (size_t)(K / 256) * qdot_block_bytes(type);
}

size_t qdot_q8_1_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 32 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return 0;
  return (size_t)M * (size_t)(K / 32) * 36;
}

size_t qdot_isum_count(int type, int64_t N, int64_t K, int64_t M) {
  if (check_dims(type, N, K, M)) return 0;
  return (size_t)M * (size_t)N * (size_t)(K / sub_len(type));
}

int qdot_quantize_q8_1(const float* x, int64_t M, int64_t K, void* x_q8, void* stream) {
  if (!x || !x_q8) return QDOT_E_ARG;
  if (M < 1 || K < 32 || K % 32 != 0 || M > kMaxDim || K > kMaxDim) return QDOT_E_ARG;
  if ((double)M * (double)K > 4.0e18) return QDOT_E_ARG;
  if (!aligned4(x) || !aligned4(x_q8)) return QDOT_E_ALIGN;
  int rc = qdot::launch_quantize_q8_1(x, M, K, x_q8, static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

int qdot_rmsnorm_quantize_q8_1(const float* x, const float* w, float eps, int64_t M, int64_t K,
                               void* x_q8, void* stream) {
  if (!x || !w || !x_q8) return QDOT_E_ARG;
  if (M < 1 || M > kMaxDim || K < 32 || K % 32 != 0 || K > QDOT_RMSNORM_MAX_K) return QDOT_E_ARG;
  if (!(eps >= 0.0f) || eps > 3.4e38f) return QDOT_E_ARG;  // also rejects NaN
  if (!aligned4(x) || !aligned4(w) || !aligned4(x_q8)) return QDOT_E_ALIGN;
  int rc = qdot::launch_rmsnorm_q8_1(x, w, eps, M, K, x_q8, static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

int qdot_qmatmul(const void* W, int type, int64_t N, int64_t K, const void* x_q8, int64_t M,
                 float* y, void* stream) {
  return run_qmatmul(W, type, N, K, x_q8, M, y, nullptr, stream, false);
}

int qdot_qmatmul_dump_isums(const void* W, int type, int64_t N, int64_t K, const void* x_q8,
                            int64_t M, float* y, int32_t* isums, void* stream) {
  return run_qmatmul(W, type, N, K, x_q8, M, y, isums, stream, true);
}

int qdot_qmatmul_multi(int n, const void* const* W, const int* types, const int64_t* N, int64_t K,
                       const void* x_q8, int64_t M, float* const* y, void* stream) {
  if (n < 1 || n > QDOT_MULTI_MAX || !W || !types || !N || !y || !x_q8) return QDOT_E_ARG;
  for (int i = 0; i < n; ++i) {
    const int st = check_dims(types[i], N[i], K, M);
    if (st) return st;
    if (!W[i] || !y[i]) return QDOT_E_ARG;
  }
  if (!aligned4(x_q8)) return QDOT_E_ALIGN;
  for (int i = 0; i < n; ++i)
    if (!aligned4(y[i])) return QDOT_E_ALIGN;
  if (M > 8) {  // mid-batch and prefill: one launch per matrix
    for (int i = 0; i < n; ++i) {
      const int st = run_qmatmul(W[i], types[i], N[i], K, x_q8, M, y[i], nullptr, stream, false);
      if (st) return st;
    }
    return QDOT_OK;
  }
  int n32[QDOT_MULTI_MAX];
  for (int i = 0; i < n; ++i) n32[i] = (int)N[i];
  const int rc = qdot::launch_qmv_multi(n, W, types, n32, (int)K, x_q8, (int)M, y, false,
                                        static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

int qdot_quantize_qmatmul(const void* W, int type, int64_t N, int64_t K, const float* x, int64_t M,
                          float* y, void* stream) {
  const int st = check_dims(type, N, K, M);
  if (st) return st;
  if (!W || !x || !y || M > QDOT_QUANTIZE_QMATMUL_MAX_M) return QDOT_E_ARG;
  if ((double)M * (double)K > 4.0e18) return QDOT_E_ARG;
  if (!aligned4(x) || !aligned4(y)) return QDOT_E_ALIGN;
  const int rc = qdot::launch_qmv_x(W, type, (int)N, (int)K, x, (int)M, y, static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

int qdot_quantize_qmatmul_multi(int n, const void* const* W, const int* types, const int64_t* N, int64_t K,
                                const float* x, int64_t M, float* const* y, void* stream) {
  if (n < 1 || n > QDOT_MULTI_MAX || !W || !types || !N || !y || !x) return QDOT_E_ARG;
  if (M > QDOT_QUANTIZE_QMATMUL_MAX_M) return QDOT_E_ARG;
  for (int i = 0; i < n; ++i) {
    const int st = check_dims(types[i], N[i], K, M);
    if (st) return st;
    if (!W[i] || !y[i]) return QDOT_E_ARG;
  }
  if (!aligned4(x)) return QDOT_E_ALIGN;
  for (int i = 0; i < n; ++i)
    if (!aligned4(y[i])) return QDOT_E_ALIGN;
  int n32[QDOT_MULTI_MAX];
  for (int i = 0; i < n; ++i) n32[i] = (int)N[i];
  const int rc = qdot::launch_qmv_multi(n, W, types, n32, (int)K, x, (int)M, y, true,
                                        static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

const char* qdot_status_str(int status) {
  switch (status) {
    case QDOT_OK: return "ok";
    case QDOT_E_ARG: return "invalid argument";
    case QDOT_E_ALIGN: return "misaligned pointer";
    case QDOT_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* qdot_kernel_name(int type, int64_t M) {
  static const char* const dec[5][8] = {
      {"qmv_dot4<Q4_K,1>", "qmv_dot4<Q4_K,2>", "qmv_dot4<Q4_K,3>", "qmv_dot4<Q4_K,4>",
       "qmv_dot4<Q4_K,5>", "qmv_dot4<Q4_K,6>", "qmv_mfma<Q4_K,7>", "qmv_mfma<Q4_K,8>"},
      {"qmv_dot4<Q6_K,1>", "qmv_dot4<Q6_K,2>", "qmv_dot4<Q6_K,3>", "qmv_dot4<Q6_K,4>",
       "qmv_dot4<Q6_K,5>", "qmv_dot4<Q6_K,6>", "qmv_mfma<Q6_K,7>", "qmv_mfma<Q6_K,8>"},
      {"qmv_dot4<IQ4_XS,1>", "qmv_dot4<IQ4_XS,2>", "qmv_dot4<IQ4_XS,3>", "qmv_dot4<IQ4_XS,4>",
       "qmv_mfma<IQ4_XS,5>", "qmv_mfma<IQ4_XS,6>", "qmv_mfma<IQ4_XS,7>", "qmv_mfma<IQ4_XS,8>"},
      {"qmv_dot4<Q4_0,1>", "qmv_dot4<Q4_0,2>", "qmv_dot4<Q4_0,3>", "qmv_dot4<Q4_0,4>",
       "qmv_dot4<Q4_0,5>", "qmv_dot4<Q4_0,6>", "qmv_dot4<Q4_0,7>", "qmv_dot4<Q4_0,8>"},
      {"qmv_dot4<Q8_0,1>", "qmv_dot4<Q8_0,2>", "qmv_dot4<Q8_0,3>", "qmv_dot4<Q8_0,4>",
       "qmv_dot4<Q8_0,5>", "qmv_dot4<Q8_0,6>", "qmv_dot4<Q8_0,7>", "qmv_dot4<Q8_0,8>"}};
  static const char* const dec16[2][8] = {
      {"qmv_mfma<Q4_K,9>", "qmv_mfma<Q4_K,10>", "qmv_mfma<Q4_K,11>", "qmv_mfma<Q4_K,12>",
       "qmv_mfma<Q4_K,13>", "qmv_mfma<Q4_K,14>", "qmv_mfma<Q4_K,15>", "qmv_mfma<Q4_K,16>"},
      {"qmv_mfma<IQ4_XS,9>", "qmv_mfma<IQ4_XS,10>", "qmv_mfma<IQ4_XS,11>", "qmv_mfma<IQ4_XS,12>",
       "qmv_mfma<IQ4_XS,13>", "qmv_mfma<IQ4_XS,14>", "qmv_mfma<IQ4_XS,15>", "qmv_mfma<IQ4_XS,16>"}};
  static const char* const mid[5] = {"qmm_skinny<Q4_K>", "qmm_skinny<Q6_K>", "qmm_skinny<IQ4_XS>",
                                     "qmm_skinny<Q4_0>", "qmm_skinny<Q8_0>"};
  static const char* const pre[5] = {"qmm_mfma<Q4_K>", "qmm_mfma<Q6_K>", "qmm_mfma<IQ4_XS>",
                                     "qmm_mfma<Q4_0>", "qmm_mfma<Q8_0>"};
  if (type < QDOT_Q4_K || type > QDOT_Q8_0 || M < 1 || M > kMaxDim) return "invalid";
  if (M <= 8) return dec[type - 1][M - 1];
  if (M <= 16 && (type == QDOT_Q4_K || type == QDOT_IQ4_XS)) return dec16[type == QDOT_Q4_K ? 0 : 1][M - 9];
  return M <= QDOT_SKINNY_MAX_M ? mid[type - 1] : pre[type - 1];
}

const char* qdot_kernel_name_shape(int type, int64_t N, int64_t K, int64_t M) {
  if (check_dims(type, N, K, M) != QDOT_OK) return "invalid";
  if (M <= 8 || (M <= 16 && (type == QDOT_Q4_K || type == QDOT_IQ4_XS))) return qdot_kernel_name(type, M);
  // the mid-batch or the prefill name of the type
  return qdot_kernel_name(type, M <= mid_max_m(type, N, K) ? QDOT_SKINNY_MAX_M : QDOT_SKINNY_MAX_M + 1);
}

const char* qdot_multi_kernel_name(int n, const int* types, const int64_t* N, int64_t K, int64_t M, int i) {
  if (n < 1 || n > QDOT_MULTI_MAX || !types || !N || i < 0 || i >= n) return "invalid";
  for (int j = 0; j < n; ++j)
    if (check_dims(types[j], N[j], K, M) != QDOT_OK) return "invalid";
  if (M > 8) return qdot_kernel_name_shape(types[i], N[i], K, M);
  static const char* const dot4[5][8] = {
      {"qmv_dot4<Q4_K,1>", "qmv_dot4<Q4_K,2>", "qmv_dot4<Q4_K,3>", "qmv_dot4<Q4_K,4>",
       "qmv_dot4<Q4_K,5>", "qmv_dot4<Q4_K,6>", "qmv_dot4<Q4_K,7>", "qmv_dot4<Q4_K,8>"},
      {"qmv_dot4<Q6_K,1>", "qmv_dot4<Q6_K,2>", "qmv_dot4<Q6_K,3>", "qmv_dot4<Q6_K,4>",
       "qmv_dot4<Q6_K,5>", "qmv_dot4<Q6_K,6>", "qmv_mfma<Q6_K,7>", "qmv_mfma<Q6_K,8>"},
      {"qmv_dot4<IQ4_XS,1>", "qmv_dot4<IQ4_XS,2>", "qmv_dot4<IQ4_XS,3>", "qmv_dot4<IQ4_XS,4>",
       "qmv_dot4<IQ4_XS,5>", "qmv_dot4<IQ4_XS,6>", "qmv_dot4<IQ4_XS,7>", "qmv_dot4<IQ4_XS,8>"},
      {"qmv_dot4<Q4_0,1>", "qmv_dot4<Q4_0,2>", "qmv_dot4<Q4_0,3>", "qmv_dot4<Q4_0,4>",
       "qmv_dot4<Q4_0,5>", "qmv_dot4<Q4_0,6>", "qmv_dot4<Q4_0,7>", "qmv_dot4<Q4_0,8>"},
      {"qmv_dot4<Q8_0,1>", "qmv_dot4<Q8_0,2>", "qmv_dot4<Q8_0,3>", "qmv_dot4<Q8_0,4>",
       "qmv_dot4<Q8_0,5>", "qmv_dot4<Q8_0,6>", "qmv_dot4<Q8_0,7>", "qmv_dot4<Q8_0,8>"}};
  static const char* const mfma[2][8] = {
      {"qmv_mfma<Q4_K,1>", "qmv_mfma<Q4_K,2>", "qmv_mfma<Q4_K,3>", "qmv_mfma<Q4_K,4>",
       "qmv_mfma<Q4_K,5>", "qmv_mfma<Q4_K,6>", "qmv_mfma<Q4_K,7>", "qmv_mfma<Q4_K,8>"},
      {"qmv_mfma<IQ4_XS,1>", "qmv_mfma<IQ4_XS,2>", "qmv_mfma<IQ4_XS,3>", "qmv_mfma<IQ4_XS,4>",
       "qmv_mfma<IQ4_XS,5>", "qmv_mfma<IQ4_XS,6>", "qmv_mfma<IQ4_XS,7>", "qmv_mfma<IQ4_XS,8>"}};
  int n32[QDOT_MULTI_MAX];
  for (int j = 0; j < n; ++j) n32[j] = (int)N[j];
  if (qdot::qmv_multi_uses_mfma(n, types, n32, (int)K, (int)M, i))
    return mfma[types[i] == QDOT_Q4_K ? 0 : 1][M - 1];
  return dot4[types[i] - 1][M - 1];
}

int qdot_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0) return QDOT_E_ARG;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || !aligned4(sink)) return QDOT_E_ALIGN;
  int rc = qdot::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

const char* qdot_build_id(void) { return "libqdot gfx950 " __DATE__ " " __TIME__; }

}  // extern "C"
