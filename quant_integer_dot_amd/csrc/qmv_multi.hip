// qmv_multi.hip -- one decode launch (M = 1..8) over up to four weight
// matrices that read the same activation rows, e.g. the Q, K and V
// projections, or gate and up.  The per-tile code is the single-matrix
// kernel's (qmv_kernel.hpp), so each output is bitwise what a launch of its
// matrix alone gives; what the group saves is the fixed cost of the launches
// it replaces (about 1.75 us of dispatch each on MI355X, plus the ramp-up and
// tail of each grid).
#include "qdot.h"
#include "qmv_kernel.hpp"

namespace qdot {

static_assert(QMV_MULTI_MAX == QDOT_MULTI_MAX, "group size of the C ABI");

template <int TA, int TB, int M, int DEPTH, bool MF, bool XF>
static int launch_multi_k(const QmvMulti& a, int K, const uint8_t* xq, hipStream_t s) {
  const int P = qmv_waves(K / QK);
  const size_t la = qmv_lds_bytes_tile<M>(qmf_group_ok<TA, M, MF>(), P);
  const size_t lb = qmv_lds_bytes_tile<M>(qmf_group_ok<TB, M, MF>(), P);
  const size_t lds = la > lb ? la : lb;
  hipLaunchKernelGGL((qmv_multi_kernel<TA, TB, M, DEPTH, MF, XF>), dim3(a.tile_end[a.n - 1]), dim3(64 * P),
                     lds, s, a, K, xq);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int TA, int TB, int M, bool MF, bool XF>
static int launch_multi_d(const QmvMulti& a, int K, const uint8_t* xq, int depth, hipStream_t s) {
  constexpr bool wide = TA == Q6_K || TA == Q8_0 || TB == Q6_K || TB == Q8_0;
  if (depth == 1) return launch_multi_k<TA, TB, M, 1, MF, XF>(a, K, xq, s);
  if constexpr (!wide && !qmf_group_ok<TA, M, MF>() && !qmf_group_ok<TB, M, MF>()) {
    if (depth == 4) return launch_multi_k<TA, TB, M, 4, MF, XF>(a, K, xq, s);
  }
  return launch_multi_k<TA, TB, M, 2, MF, XF>(a, K, xq, s);
}

template <int TA, int TB, int M, bool XF>
static int launch_multi_f(const QmvMulti& a, int K, const uint8_t* xq, int depth, bool mf, hipStream_t s) {
  if constexpr (!XF && (qmf_type<TA>() || qmf_type<TB>())) {
    if (mf) return launch_multi_d<TA, TB, M, true, false>(a, K, xq, depth, s);
  }
  return launch_multi_d<TA, TB, M, false, XF>(a, K, xq, depth, s);
}

template <int TA, int TB, bool XF>
static int launch_multi_m(const QmvMulti& a, int K, const uint8_t* xq, int M, int depth, bool mf,
                          hipStream_t s) {
  switch (M) {
    case 1: return launch_multi_f<TA, TB, 1, XF>(a, K, xq, depth, mf, s);
    case 2: return launch_multi_f<TA, TB, 2, XF>(a, K, xq, depth, mf, s);
    case 3: return launch_multi_f<TA, TB, 3, XF>(a, K, xq, depth, mf, s);
    case 4: return launch_multi_f<TA, TB, 4, XF>(a, K, xq, depth, mf, s);
    case 5: return launch_multi_f<TA, TB, 5, XF>(a, K, xq, depth, mf, s);
    case 6: return launch_multi_f<TA, TB, 6, XF>(a, K, xq, depth, mf, s);
    case 7: return launch_multi_f<TA, TB, 7, XF>(a, K, xq, depth, mf, s);
    case 8: return launch_multi_f<TA, TB, 8, XF>(a, K, xq, depth, mf, s);
    default: return -2;
  }
}

// Whether the group idx[0..cnt-1] (types ta, tb) runs MFMA tiles for its
// Q4_K / IQ4_XS matrices (measured, see qmv_kernel.hpp): with K >= 4096, from
// M = 3, and at any M for groups under 4 MB per stage (q+k+v).  At K = 1536
// (six superblocks a row) the dot4 tile stays faster.
static bool group_mfma(const int* idx, int cnt, const int* types, const int* N, int K, int M, int ta,
                       int tb, long* stage_out) {
  long stage = 0;
  for (int g = 0; g < cnt; ++g) stage += qmv_stage_bytes(types[idx[g]], N[idx[g]], K);
  if (stage_out) *stage_out = stage;
  return (ta == Q4_K || tb == Q4_K || ta == IQ4_XS || tb == IQ4_XS) && K >= 4096 &&
         (M >= 3 || stage < (4L << 20));
}

// The fused type mixes of GGUF's usual mixed-precision files: Q4_K with Q6_K
// and Q4_0 with Q8_0.  Any other mix runs one launch per weight type.
static bool fused_mix(int nd, const int* distinct) {
  return nd == 1 || (nd == 2 && ((distinct[0] == Q4_K && distinct[1] == Q6_K) ||
                                 (distinct[0] == Q6_K && distinct[1] == Q4_K) ||
                                 (distinct[0] == Q4_0 && distinct[1] == Q8_0) ||
                                 (distinct[0] == Q8_0 && distinct[1] == Q4_0)));
}

template <bool XF>
static int launch_types(const QmvMulti& a, int K, const uint8_t* x8, int M, int depth, bool mf, int ta,
                        int tb, hipStream_t s) {
  if (ta == tb) {
    switch (ta) {
      case Q4_K: return launch_multi_m<Q4_K, Q4_K, XF>(a, K, x8, M, depth, mf, s);
      case Q6_K: return launch_multi_m<Q6_K, Q6_K, XF>(a, K, x8, M, depth, mf, s);
      case IQ4_XS: return launch_multi_m<IQ4_XS, IQ4_XS, XF>(a, K, x8, M, depth, mf, s);
      case Q4_0: return launch_multi_m<Q4_0, Q4_0, XF>(a, K, x8, M, depth, mf, s);
      case Q8_0: return launch_multi_m<Q8_0, Q8_0, XF>(a, K, x8, M, depth, mf, s);
      default: return -2;
    }
  }
  if (ta == Q4_K && tb == Q6_K) return launch_multi_m<Q4_K, Q6_K, XF>(a, K, x8, M, depth, mf, s);
  if (ta == Q4_0 && tb == Q8_0) return launch_multi_m<Q4_0, Q8_0, XF>(a, K, x8, M, depth, mf, s);
  return -2;
}

// One launch over the matrices idx[0..cnt-1] (all of type ta or tb).  xf:
// xq holds fp32 activations, quantized in the kernel (dot4 tiles).
static int launch_group(const int* idx, int cnt, const void* const* W, const int* types, const int* N,
                        int K, const void* xq, int M, float* const* y, int ta, int tb, bool xf,
                        hipStream_t s) {
  QmvMulti a{};
  long stage = 0;
  const bool mf = !xf && group_mfma(idx, cnt, types, N, K, M, ta, tb, &stage);
  if (xf)
    for (int g = 0; g < cnt; ++g) stage += qmv_stage_bytes(types[idx[g]], N[idx[g]], K);
  int tiles = 0;
  for (int g = 0; g < cnt; ++g) {
    const int i = idx[g];
    a.W[g] = static_cast<const uint8_t*>(W[i]);
    a.y[g] = y[i];
    a.N[g] = N[i];
    a.type[g] = types[i];
    const int rows = qmv_rows(types[i], mf);
    tiles += (N[i] + rows - 1) / rows;
    if (tiles > 0x7FFFFFFF / 2) return -1;
    a.tile_end[g] = tiles;
  }
  a.n = cnt;
  const bool wide = ta == Q6_K || ta == Q8_0 || tb == Q6_K || tb == Q8_0;
  const int depth = mf ? qmf_depth(stage) : qmv_depth_for(stage, M, wide);
  const uint8_t* x8 = static_cast<const uint8_t*>(xq);
  if (xf) return launch_types<true>(a, K, x8, M, depth, false, ta, tb, s);
  return launch_types<false>(a, K, x8, M, depth, mf, ta, tb, s);
}

static int distinct_types(int n, const int* types, int* distinct) {
  int nd = 0;
  for (int i = 0; i < n; ++i) {
    bool seen = false;
    for (int d = 0; d < nd; ++d) seen = seen || distinct[d] == types[i];
    if (!seen) distinct[nd++] = types[i];
  }
  return nd;
}

// Whether matrix i of a grouped call runs the MFMA tile (else the dot4 tile):
// the decision of the launch that holds it.
bool qmv_multi_uses_mfma(int n, const int* types, const int* N, int K, int M, int i) {
  if (types[i] != Q4_K && types[i] != IQ4_XS) return false;
  int distinct[QMV_MULTI_MAX];
  const int nd = distinct_types(n, types, distinct);
  int idx[QMV_MULTI_MAX];
  int cnt = 0, ta, tb;
  if (fused_mix(nd, distinct)) {
    for (int j = 0; j < n; ++j) idx[cnt++] = j;
    ta = distinct[0];
    tb = nd == 2 ? distinct[1] : distinct[0];
  } else {
    for (int j = 0; j < n; ++j)
      if (types[j] == types[i]) idx[cnt++] = j;
    ta = tb = types[i];
  }
  return group_mfma(idx, cnt, types, N, K, M, ta, tb, nullptr);
}

int launch_qmv_multi(int n, const void* const* W, const int* types, const int* N, int K, const void* xq,
                     int M, float* const* y, bool xf, hipStream_t s) {
  int distinct[QMV_MULTI_MAX];
  const int nd = distinct_types(n, types, distinct);
  int idx[QMV_MULTI_MAX];
  if (fused_mix(nd, distinct)) {
    for (int i = 0; i < n; ++i) idx[i] = i;
    int ta = distinct[0], tb = nd == 2 ? distinct[1] : distinct[0];
    if (ta > tb) { const int t = ta; ta = tb; tb = t; }
    return launch_group(idx, n, W, types, N, K, xq, M, y, ta, tb, xf, s);
  }
  for (int d = 0; d < nd; ++d) {
    int cnt = 0;
    for (int i = 0; i < n; ++i)
      if (types[i] == distinct[d]) idx[cnt++] = i;
    const int rc = launch_group(idx, cnt, W, types, N, K, xq, M, y, distinct[d], distinct[d], xf, s);
    if (rc) return rc;
  }
  return 0;
}

}  // namespace qdot
