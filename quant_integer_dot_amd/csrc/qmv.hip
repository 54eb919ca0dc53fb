// qmv.hip -- launches of the decode kernel (M = 1..8; Q4_K and IQ4_XS up to
// M = 16) for one matrix; the kernel is in qmv_kernel.hpp.
#include "qmv_kernel.hpp"

namespace qdot {

template <int T, int M, int DEPTH, bool DUMP>
static int launch_qmv_k(const uint8_t* W, int N, int K, const uint8_t* xq, float* y, int32_t* isums,
                        hipStream_t s) {
  const int P = qmv_waves(K / QK);
  const size_t lds = qmv_lds_bytes<T, M>(P);
  constexpr int ROWS = qmv_tile_rows<T, M>();
  const int grid = (N + ROWS - 1) / ROWS;
  hipLaunchKernelGGL((qmv_kernel<T, M, DEPTH, DUMP>), dim3(grid), dim3(64 * P), lds, s, W, N, K, xq,
                     y, isums);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int T, int M, bool DUMP>
static int launch_qmv_r(const uint8_t* W, int N, int K, const uint8_t* xq, float* y,
                        int32_t* isums, hipStream_t s) {
  // 16-row MFMA tiles (M = 9..16): the depth rule of the 8-row tile; the
  // debug dump keeps one superblock in flight (fewer registers to spill)
  if constexpr (M > 8) {
    if constexpr (!DUMP)
      if (qmf_depth(qmv_stage_bytes(T, N, K)) == 2) return launch_qmv_k<T, M, 2, false>(W, N, K, xq, y, isums, s);
    return launch_qmv_k<T, M, 1, DUMP>(W, N, K, xq, y, isums, s);
  } else if constexpr (DUMP) {
    return launch_qmv_k<T, M, 2, true>(W, N, K, xq, y, isums, s);
  } else {
    switch (qmf_ok<T, M>() ? qmf_depth(qmv_stage_bytes(T, N, K)) : qmv_depth(T, M, N, K)) {
      case 1: return launch_qmv_k<T, M, 1, false>(W, N, K, xq, y, isums, s);
      case 2: return launch_qmv_k<T, M, 2, false>(W, N, K, xq, y, isums, s);
      default:
        if constexpr (T == Q6_K || T == Q8_0 || qmf_ok<T, M>())
          return launch_qmv_k<T, M, 2, false>(W, N, K, xq, y, isums, s);
        else return launch_qmv_k<T, M, 4, false>(W, N, K, xq, y, isums, s);
    }
  }
}

template <int T, bool DUMP>
static int launch_qmv_m(const uint8_t* W, int N, int K, const uint8_t* xq, int M, float* y,
                        int32_t* isums, hipStream_t s) {
  switch (M) {
    case 1: return launch_qmv_r<T, 1, DUMP>(W, N, K, xq, y, isums, s);
    case 2: return launch_qmv_r<T, 2, DUMP>(W, N, K, xq, y, isums, s);
    case 3: return launch_qmv_r<T, 3, DUMP>(W, N, K, xq, y, isums, s);
    case 4: return launch_qmv_r<T, 4, DUMP>(W, N, K, xq, y, isums, s);
    case 5: return launch_qmv_r<T, 5, DUMP>(W, N, K, xq, y, isums, s);
    case 6: return launch_qmv_r<T, 6, DUMP>(W, N, K, xq, y, isums, s);
    case 7: return launch_qmv_r<T, 7, DUMP>(W, N, K, xq, y, isums, s);
    case 8: return launch_qmv_r<T, 8, DUMP>(W, N, K, xq, y, isums, s);
    default: break;
  }
  if constexpr (qmf_type<T>()) {  // M = 9..16 on the MFMA tile
    switch (M) {
      case 9: return launch_qmv_r<T, 9, DUMP>(W, N, K, xq, y, isums, s);
      case 10: return launch_qmv_r<T, 10, DUMP>(W, N, K, xq, y, isums, s);
      case 11: return launch_qmv_r<T, 11, DUMP>(W, N, K, xq, y, isums, s);
      case 12: return launch_qmv_r<T, 12, DUMP>(W, N, K, xq, y, isums, s);
      case 13: return launch_qmv_r<T, 13, DUMP>(W, N, K, xq, y, isums, s);
      case 14: return launch_qmv_r<T, 14, DUMP>(W, N, K, xq, y, isums, s);
      case 15: return launch_qmv_r<T, 15, DUMP>(W, N, K, xq, y, isums, s);
      case 16: return launch_qmv_r<T, 16, DUMP>(W, N, K, xq, y, isums, s);
      default: break;
    }
  }
  return -2;
}

// In-kernel quantization (fp32 activations x; dot4 tile, M = 1..8).
template <int T, int M, int DEPTH>
static int launch_qmv_xk(const uint8_t* W, int N, int K, const uint8_t* x, float* y, hipStream_t s) {
  const int P = qmv_waves(K / QK);
  const size_t lds = qmv_lds_bytes_tile<M>(false, P);
  const int grid = (N + QMV_SLOTS - 1) / QMV_SLOTS;
  hipLaunchKernelGGL((qmv_kernel<T, M, DEPTH, false, true>), dim3(grid), dim3(64 * P), lds, s, W, N, K, x,
                     y, nullptr);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int T, int M>
static int launch_qmv_xr(const uint8_t* W, int N, int K, const uint8_t* x, float* y, hipStream_t s) {
  switch (qmv_depth(T, M, N, K)) {
    case 1: return launch_qmv_xk<T, M, 1>(W, N, K, x, y, s);
    case 2: return launch_qmv_xk<T, M, 2>(W, N, K, x, y, s);
    default:
      if constexpr (T == Q6_K || T == Q8_0) return launch_qmv_xk<T, M, 2>(W, N, K, x, y, s);
      else return launch_qmv_xk<T, M, 4>(W, N, K, x, y, s);
  }
}

template <int T>
static int launch_qmv_xm(const uint8_t* W, int N, int K, const uint8_t* x, int M, float* y, hipStream_t s) {
  switch (M) {
    case 1: return launch_qmv_xr<T, 1>(W, N, K, x, y, s);
    case 2: return launch_qmv_xr<T, 2>(W, N, K, x, y, s);
    case 3: return launch_qmv_xr<T, 3>(W, N, K, x, y, s);
    case 4: return launch_qmv_xr<T, 4>(W, N, K, x, y, s);
    case 5: return launch_qmv_xr<T, 5>(W, N, K, x, y, s);
    case 6: return launch_qmv_xr<T, 6>(W, N, K, x, y, s);
    case 7: return launch_qmv_xr<T, 7>(W, N, K, x, y, s);
    case 8: return launch_qmv_xr<T, 8>(W, N, K, x, y, s);
    default: return -2;
  }
}

int launch_qmv_x(const void* W, int type, int N, int K, const float* x, int M, float* y, hipStream_t s) {
  const uint8_t* w8 = static_cast<const uint8_t*>(W);
  const uint8_t* x8 = reinterpret_cast<const uint8_t*>(x);
  switch (type) {
    case Q4_K: return launch_qmv_xm<Q4_K>(w8, N, K, x8, M, y, s);
    case Q6_K: return launch_qmv_xm<Q6_K>(w8, N, K, x8, M, y, s);
    case IQ4_XS: return launch_qmv_xm<IQ4_XS>(w8, N, K, x8, M, y, s);
    case Q4_0: return launch_qmv_xm<Q4_0>(w8, N, K, x8, M, y, s);
    case Q8_0: return launch_qmv_xm<Q8_0>(w8, N, K, x8, M, y, s);
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
    case Q4_0:
      return dump ? launch_qmv_m<Q4_0, true>(w8, N, K, x8, M, y, isums, s)
                  : launch_qmv_m<Q4_0, false>(w8, N, K, x8, M, y, isums, s);
    case Q8_0:
      return dump ? launch_qmv_m<Q8_0, true>(w8, N, K, x8, M, y, isums, s)
                  : launch_qmv_m<Q8_0, false>(w8, N, K, x8, M, y, isums, s);
    default:
      return -2;
  }
}

}  // namespace qdot
