// qmm.hip -- launches of the prefill kernel (M > 8).  The kernel itself is
// in qmm_kernel.hpp; this file is built with MFMA results in VGPRs, the
// sub-block-sum dump variant in qmm_dump.hip without that option.
#include "qmm_kernel.hpp"

namespace qdot {

int launch_qmm_dump(const uint8_t* W, int type, int N, int K, const uint8_t* xq, int M, float* y,
                    int32_t* isums, hipStream_t s);

int launch_qmm(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s) {
  const uint8_t* w8 = static_cast<const uint8_t*>(W);
  const uint8_t* x8 = static_cast<const uint8_t*>(xq);
  if (isums != nullptr) return launch_qmm_dump(w8, type, N, K, x8, M, y, isums, s);
  switch (type) {
    case Q4_K: return launch_qmm_t<Q4_K, false>(w8, N, K, x8, M, y, nullptr, s);
    case Q6_K: return launch_qmm_t<Q6_K, false>(w8, N, K, x8, M, y, nullptr, s);
    case IQ4_XS: return launch_qmm_t<IQ4_XS, false>(w8, N, K, x8, M, y, nullptr, s);
    case Q4_0: return launch_qmm_t<Q4_0, false>(w8, N, K, x8, M, y, nullptr, s);
    case Q8_0: return launch_qmm_t<Q8_0, false>(w8, N, K, x8, M, y, nullptr, s);
    default: return -2;
  }
}

}  // namespace qdot
