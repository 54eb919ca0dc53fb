"""Thin ctypes binding over libqdot.so (declared in include/qdot.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  Arguments may be torch tensors (their data_ptr is
passed) or plain integer addresses.  The stream defaults to torch's current
stream on the tensor's device.  There is no fallback: if the library is
missing, every call raises.
"""
import ctypes
import os

QDOT_Q4_K, QDOT_Q6_K, QDOT_IQ4_XS, QDOT_Q4_0, QDOT_Q8_0 = 1, 2, 3, 4, 5
QDOT_OK, QDOT_E_ARG, QDOT_E_ALIGN, QDOT_E_HIP = 0, -1, -2, -3
QDOT_ATTN_NOALLOC_BYTES = 16 << 20   # include/qdot.h

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libqdot.so"
_lib = None


class QdotError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {qdot_status_str(status)} ({status})")


def library_path():
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load libqdot.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: the HIP library has not been built "
            "(run __graft_entry__.build()); there is no fallback path")
    L = ctypes.CDLL(path)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.qdot_block_bytes.argtypes = [i32]
    L.qdot_block_bytes.restype = ctypes.c_size_t
    L.qdot_weight_bytes.argtypes = [i32, i64, i64]
    L.qdot_weight_bytes.restype = ctypes.c_size_t
    L.qdot_q8_1_bytes.argtypes = [i64, i64]
    L.qdot_q8_1_bytes.restype = ctypes.c_size_t
    L.qdot_isum_count.argtypes = [i32, i64, i64, i64]
    L.qdot_isum_count.restype = ctypes.c_size_t
    L.qdot_quantize_q8_1.argtypes = [P, i64, i64, P, P]
    L.qdot_quantize_q8_1.restype = i32
    L.qdot_qmatmul.argtypes = [P, i32, i64, i64, P, i64, P, P]
    L.qdot_qmatmul.restype = i32
    L.qdot_qmatmul_dump_isums.argtypes = [P, i32, i64, i64, P, i64, P, P, P]
    L.qdot_qmatmul_dump_isums.restype = i32
    L.qdot_qmatmul_multi.argtypes = [i32, ctypes.POINTER(P), ctypes.POINTER(i32), ctypes.POINTER(i64),
                                     i64, P, i64, ctypes.POINTER(P), P]
    L.qdot_qmatmul_multi.restype = i32
    L.qdot_quantize_qmatmul.argtypes = [P, i32, i64, i64, P, i64, P, P]
    L.qdot_quantize_qmatmul.restype = i32
    L.qdot_quantize_qmatmul_multi.argtypes = [i32, ctypes.POINTER(P), ctypes.POINTER(i32), ctypes.POINTER(i64),
                                              i64, P, i64, ctypes.POINTER(P), P]
    L.qdot_quantize_qmatmul_multi.restype = i32
    L.qdot_rmsnorm_quantize_q8_1.argtypes = [P, P, ctypes.c_float, i64, i64, P, P]
    L.qdot_rmsnorm_quantize_q8_1.restype = i32
    L.qdot_attn_decode_kv4.argtypes = [P, i64, P, P, i64, i64, i64, ctypes.c_float, P, P, ctypes.c_size_t, P]
    L.qdot_attn_decode_kv4.restype = i32
    L.qdot_attn_decode_kv4_noalloc.argtypes = [P, i64, P, P, i64, i64, i64, ctypes.c_float, P, P]
    L.qdot_attn_decode_kv4_noalloc.restype = i32
    L.qdot_attn_kv4_row_bytes.argtypes = [i64]
    L.qdot_attn_kv4_row_bytes.restype = ctypes.c_size_t
    L.qdot_attn_kv4_workspace_bytes.argtypes = [i64, i64]
    L.qdot_attn_kv4_workspace_bytes.restype = ctypes.c_size_t
    L.qdot_status_str.argtypes = [i32]
    L.qdot_status_str.restype = ctypes.c_char_p
    L.qdot_kernel_name.argtypes = [i32, i64]
    L.qdot_kernel_name.restype = ctypes.c_char_p
    L.qdot_kernel_name_shape.argtypes = [i32, i64, i64, i64]
    L.qdot_kernel_name_shape.restype = ctypes.c_char_p
    L.qdot_multi_kernel_name.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i64), i64, i64, i32]
    L.qdot_multi_kernel_name.restype = ctypes.c_char_p
    L.qdot_stream_read.argtypes = [P, i64, P, P]
    L.qdot_stream_read.restype = i32
    L.qdot_build_id.argtypes = []
    L.qdot_build_id.restype = ctypes.c_char_p
    _lib = L
    return L


def _addr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream, *tensors):
    """Raw hipStream_t: explicit int/None-as-default, else torch's current."""
    if stream is not None:
        if isinstance(stream, int):
            return stream
        return stream.cuda_stream
    for t in tensors:
        if hasattr(t, "device") and getattr(t.device, "type", None) == "cuda":
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return 0


def _check(status, where):
    if status != QDOT_OK:
        raise QdotError(status, where)


def qdot_block_bytes(wtype):
    return load().qdot_block_bytes(wtype)


def qdot_weight_bytes(wtype, N, K):
    return load().qdot_weight_bytes(wtype, N, K)


def qdot_q8_1_bytes(M, K):
    return load().qdot_q8_1_bytes(M, K)


def qdot_isum_count(wtype, N, K, M):
    return load().qdot_isum_count(wtype, N, K, M)


def qdot_quantize_q8_1(x, M, K, x_q8, stream=None):
    s = _stream(stream, x, x_q8)
    _check(load().qdot_quantize_q8_1(_addr(x), M, K, _addr(x_q8), s), "qdot_quantize_q8_1")


def qdot_rmsnorm_quantize_q8_1(x, w, eps, M, K, x_q8, stream=None):
    s = _stream(stream, x, w, x_q8)
    _check(load().qdot_rmsnorm_quantize_q8_1(_addr(x), _addr(w), float(eps), M, K, _addr(x_q8), s),
           "qdot_rmsnorm_quantize_q8_1")


def qdot_qmatmul(W, wtype, N, K, x_q8, M, y, stream=None):
    s = _stream(stream, W, x_q8, y)
    _check(load().qdot_qmatmul(_addr(W), wtype, N, K, _addr(x_q8), M, _addr(y), s),
           "qdot_qmatmul")


def qdot_qmatmul_multi(Ws, wtypes, Ns, K, x_q8, M, ys, stream=None):
    """One launch over several matrices sharing x_q8: ys[i] = Ws[i] x."""
    n = len(Ws)
    if not (len(wtypes) == n and len(Ns) == n and len(ys) == n):
        raise ValueError("Ws, wtypes, Ns and ys must have the same length")
    s = _stream(stream, x_q8, *Ws, *ys)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    w_arr = (P * max(n, 1))(*[_addr(w) for w in Ws])
    t_arr = (i32 * max(n, 1))(*wtypes)
    n_arr = (i64 * max(n, 1))(*Ns)
    y_arr = (P * max(n, 1))(*[_addr(y) for y in ys])
    _check(load().qdot_qmatmul_multi(n, w_arr, t_arr, n_arr, K, _addr(x_q8), M, y_arr, s),
           "qdot_qmatmul_multi")


def qdot_quantize_qmatmul(W, wtype, N, K, x, M, y, stream=None):
    """y = W x for fp32 x, the Q8_1 quantization done inside the decode kernel."""
    s = _stream(stream, W, x, y)
    _check(load().qdot_quantize_qmatmul(_addr(W), wtype, N, K, _addr(x), M, _addr(y), s),
           "qdot_quantize_qmatmul")


def qdot_quantize_qmatmul_multi(Ws, wtypes, Ns, K, x, M, ys, stream=None):
    """Grouped qdot_quantize_qmatmul over matrices sharing the fp32 activations x."""
    n = len(Ws)
    if not (len(wtypes) == n and len(Ns) == n and len(ys) == n):
        raise ValueError("Ws, wtypes, Ns and ys must have the same length")
    s = _stream(stream, x, *Ws, *ys)
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    w_arr = (P * max(n, 1))(*[_addr(w) for w in Ws])
    t_arr = (i32 * max(n, 1))(*wtypes)
    n_arr = (i64 * max(n, 1))(*Ns)
    y_arr = (P * max(n, 1))(*[_addr(y) for y in ys])
    _check(load().qdot_quantize_qmatmul_multi(n, w_arr, t_arr, n_arr, K, _addr(x), M, y_arr, s),
           "qdot_quantize_qmatmul_multi")


def qdot_qmatmul_dump_isums(W, wtype, N, K, x_q8, M, y, isums, stream=None):
    s = _stream(stream, W, x_q8, y, isums)
    _check(load().qdot_qmatmul_dump_isums(_addr(W), wtype, N, K, _addr(x_q8), M, _addr(y),
                                          _addr(isums), s), "qdot_qmatmul_dump_isums")


def qdot_attn_kv4_row_bytes(D):
    return load().qdot_attn_kv4_row_bytes(D)


def qdot_attn_kv4_workspace_bytes(Hq, T):
    return load().qdot_attn_kv4_workspace_bytes(Hq, T)


def qdot_attn_decode_kv4(q_q8, Hq, Kc, Vc, Hkv, T, D, scale, out, workspace, workspace_bytes, stream=None):
    st = _stream(stream, out)
    _check(load().qdot_attn_decode_kv4(_addr(q_q8), Hq, _addr(Kc), _addr(Vc), Hkv, T, D, float(scale),
                                        _addr(out), _addr(workspace), int(workspace_bytes), st),
           "qdot_attn_decode_kv4")


def qdot_attn_decode_kv4_noalloc(q_q8, Hq, Kc, Vc, Hkv, T, D, scale, out, stream=None):
    """qdot_attn_decode_kv4 with the library's static workspace (no allocation)."""
    st = _stream(stream, out)
    _check(load().qdot_attn_decode_kv4_noalloc(_addr(q_q8), Hq, _addr(Kc), _addr(Vc), Hkv, T, D,
                                                float(scale), _addr(out), st),
           "qdot_attn_decode_kv4_noalloc")


def qdot_status_str(status):
    try:
        return load().qdot_status_str(status).decode()
    except RuntimeError:
        return "library not loaded"


def qdot_kernel_name(wtype, M):
    return load().qdot_kernel_name(wtype, M).decode()


def qdot_kernel_name_shape(wtype, N, K, M):
    return load().qdot_kernel_name_shape(wtype, N, K, M).decode()


def qdot_multi_kernel_name(types, Ns, K, M, i):
    n = len(types)
    if len(Ns) != n:
        raise ValueError("types and Ns must have the same length")
    ta = (ctypes.c_int * n)(*types)
    na = (ctypes.c_int64 * n)(*Ns)
    return load().qdot_multi_kernel_name(n, ta, na, K, M, i).decode()


def qdot_stream_read(src, nbytes, sink, stream=None):
    """Read-only streaming reference kernel over nbytes of src (measurement)."""
    s = _stream(stream, sink)
    _check(load().qdot_stream_read(_addr(src), int(nbytes), _addr(sink), s), "qdot_stream_read")


def qdot_build_id():
    return load().qdot_build_id().decode()
