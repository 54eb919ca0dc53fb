// qmm_dump.hip -- the prefill kernel with the integer sub-block sums also
// written out (test and debug path; same arithmetic as the plain launch).
#include "qmm_kernel.hpp"

namespace qdot {

int launch_qmm_dump(const uint8_t* W, int type, int N, int K, const uint8_t* xq, int M, float* y,
                    int32_t* isums, hipStream_t s) {
  switch (type) {
    case Q4_K: return launch_qmm_t<Q4_K, true>(W, N, K, xq, M, y, isums, s);
    case Q6_K: return launch_qmm_t<Q6_K, true>(W, N, K, xq, M, y, isums, s);
    case IQ4_XS: return launch_qmm_t<IQ4_XS, true>(W, N, K, xq, M, y, isums, s);
    case Q4_0: return launch_qmm_t<Q4_0, true>(W, N, K, xq, M, y, isums, s);
    case Q8_0: return launch_qmm_t<Q8_0, true>(W, N, K, xq, M, y, isums, s);
    default: return -2;
  }
}

}  // namespace qdot
