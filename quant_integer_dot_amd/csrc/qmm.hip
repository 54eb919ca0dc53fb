// qmm.hip -- M > 8 (prefill) entry.  Placeholder until the MFMA i8 kernel:
// runs the decode kernel over 8-row chunks of the activations.
#include "qdot_common.hpp"

namespace qdot {
int launch_qmv(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s);

int launch_qmm(const void* W, int type, int N, int K, const void* xq, int M, float* y,
               int32_t* isums, hipStream_t s) {
  const int sub = type == Q6_K ? 16 : 32;
  for (int m0 = 0; m0 < M; m0 += 8) {
    const int mc = M - m0 < 8 ? M - m0 : 8;
    const uint8_t* x = static_cast<const uint8_t*>(xq) + (size_t)m0 * (K / Q8_BLOCK) * Q8_BYTES;
    int32_t* is = isums ? isums + (size_t)m0 * N * (K / sub) : nullptr;
    int rc = launch_qmv(W, type, N, K, x, mc, y + (size_t)m0 * N, is, s);
    if (rc) return rc;
  }
  return 0;
}
}  // namespace qdot
