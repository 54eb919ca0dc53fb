// api_attn.cpp -- the C ABI of the int4-KV decode attention (declared in
// include/qdot.h): argument validation before any HIP call, then the two
// launches of attn_kv4.hip on the caller's stream.  No allocation: the caller
// passes the workspace, or (qdot_attn_decode_kv4_noalloc) the workspace is
// this file's static device array.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "qdot.h"

// The workspace of qdot_attn_decode_kv4_noalloc: a file-scope device array
// (every GPU the library runs on holds its own copy until the process ends).
// In host code `scratch` is only the runtime's handle for the symbol; the
// device address of the current device's copy comes from hipGetSymbolAddress
// (scratch_address below), and only that address is ever passed to a kernel.
static __device__ __attribute__((aligned(256))) uint8_t scratch[QDOT_ATTN_NOALLOC_BYTES];

namespace qdot {
size_t attn_kv4_workspace_bytes(int64_t Hq, int64_t T);
int launch_attn_kv4(const void* q_q8, int Hq, const void* Kc, const void* Vc, int Hkv, int T, float scale,
                    float* out, void* workspace, hipStream_t s);
}  // namespace qdot

namespace {
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Everything but the workspace, checked before any HIP call.
int check_attn(const void* q_q8, int64_t Hq, const void* Kc, const void* Vc, int64_t Hkv, int64_t T,
               int64_t D, float scale, const float* out) {
  if (!q_q8 || !Kc || !Vc || !out) return QDOT_E_ARG;
  if (D != QDOT_ATTN_HEAD_DIM) return QDOT_E_ARG;
  if (Hq < 1 || Hkv < 1 || Hq > QDOT_ATTN_MAX_HEADS || Hq % Hkv != 0) return QDOT_E_ARG;
  if (Hq / Hkv > QDOT_ATTN_MAX_GROUP) return QDOT_E_ARG;
  if (T < 1 || T > QDOT_ATTN_MAX_T) return QDOT_E_ARG;
  if (!(scale == scale) || scale > 3.4e38f || scale < -3.4e38f) return QDOT_E_ARG;  // NaN, inf
  if (!aligned(Kc, 8) || !aligned(Vc, 8)) return QDOT_E_ALIGN;
  if (!aligned(q_q8, 4) || !aligned(out, 4)) return QDOT_E_ALIGN;
  return QDOT_OK;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept for the process.
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QDOT_E_HIP;
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) scratch_ptr[dev] = p;
  });
  if (!scratch_ptr[dev]) return QDOT_E_HIP;
  *out = scratch_ptr[dev];
  return QDOT_OK;
}
}  // namespace

extern "C" {

size_t qdot_attn_kv4_row_bytes(int64_t D) {
  return D >= 32 && D % 32 == 0 && D <= QDOT_ATTN_HEAD_DIM ? (size_t)(D / 32) * 18 : 0;
}

size_t qdot_attn_kv4_workspace_bytes(int64_t Hq, int64_t T) {
  if (Hq < 1 || Hq > QDOT_ATTN_MAX_HEADS || T < 1 || T > QDOT_ATTN_MAX_T) return 0;
  return qdot::attn_kv4_workspace_bytes(Hq, T);
}

int qdot_attn_decode_kv4(const void* q_q8, int64_t Hq, const void* Kc, const void* Vc, int64_t Hkv,
                         int64_t T, int64_t D, float scale, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int st = check_attn(q_q8, Hq, Kc, Vc, Hkv, T, D, scale, out);
  if (st) return st;
  if (!workspace || workspace_bytes < qdot::attn_kv4_workspace_bytes(Hq, T)) return QDOT_E_ARG;
  if (!aligned(workspace, 4)) return QDOT_E_ALIGN;
  int rc = qdot::launch_attn_kv4(q_q8, (int)Hq, Kc, Vc, (int)Hkv, (int)T, scale, out, workspace,
                                 static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

int qdot_attn_decode_kv4_noalloc(const void* q_q8, int64_t Hq, const void* Kc, const void* Vc,
                                 int64_t Hkv, int64_t T, int64_t D, float scale, float* out,
                                 void* stream) {
  const int st = check_attn(q_q8, Hq, Kc, Vc, Hkv, T, D, scale, out);
  if (st) return st;
  if (qdot::attn_kv4_workspace_bytes(Hq, T) > (size_t)QDOT_ATTN_NOALLOC_BYTES) return QDOT_E_ARG;
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa) return sa;
  // Nothing in the workspace has to start at zero: the partial kernel writes
  // every (head, chunk) entry the combine kernel reads.
  int rc = qdot::launch_attn_kv4(q_q8, (int)Hq, Kc, Vc, (int)Hkv, (int)T, scale, out, ws,
                                 static_cast<hipStream_t>(stream));
  return rc == 0 ? QDOT_OK : QDOT_E_HIP;
}

}  // extern "C"
