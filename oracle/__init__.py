"""CPU oracle for the block-quantized integer-dot matmul (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library under ``quant_integer_dot_amd``) never does: the two share no code.

This module is argument marshalling over ``liboracle.so`` (plain C, fp64), which
``build()`` compiles from ``oracle.c``.  Every function states the passage of the
pages it follows in ``oracle.c``.  The loops over independent outputs run on
several host threads (OpenMP; ``set_threads``); each output is computed by one
thread in the written order, so results do not depend on the thread count.
"""
import ctypes
import os

import numpy as np

Q4_K, Q6_K, IQ4_XS, Q4_0, Q8_0 = 1, 2, 3, 4, 5
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, IQ4_XS: 136, Q4_0: 144, Q8_0: 272}   # per 256 weights
SUBLEN = {Q4_K: 32, Q6_K: 16, IQ4_XS: 32, Q4_0: 32, Q8_0: 32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose=False):
    """Compile oracle.c into liboracle.so with the host C compiler."""
    import subprocess

    cmd = ["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH,
           os.path.join(_HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        L.oracle_quantize_q8_1.argtypes = [P, i64, i64, P]
        L.oracle_quantize_q8_1.restype = None
        L.oracle_dequant_q8_1.argtypes = [P, i64, i64, P]
        L.oracle_dequant_q8_1.restype = None
        L.oracle_dequant.argtypes = [P, ctypes.c_int, i64, i64, P]
        L.oracle_dequant.restype = ctypes.c_int
        L.oracle_isums.argtypes = [P, ctypes.c_int, i64, i64, P, i64, P]
        L.oracle_isums.restype = ctypes.c_int
        L.oracle_qmatmul.argtypes = [P, ctypes.c_int, i64, i64, P, i64, P, P, P]
        L.oracle_qmatmul.restype = ctypes.c_int
        L.oracle_qmatmul_rows.argtypes = [P, ctypes.c_int, i64, i64, P, i64, P, i64, P, P]
        L.oracle_qmatmul_rows.restype = ctypes.c_int
        L.oracle_rmsnorm.argtypes = [P, P, ctypes.c_float, i64, i64, P, P]
        L.oracle_rmsnorm.restype = None
        L.oracle_attn_decode_kv4.argtypes = [P, i64, P, P, i64, i64, i64, ctypes.c_double, P, P]
        L.oracle_attn_decode_kv4.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = None
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_codebook.argtypes = []
        L.oracle_codebook.restype = ctypes.POINTER(ctypes.c_int)
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _u8(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        a = a.view(np.uint8)
    return a


def set_threads(n):
    """Host threads for the loops over outputs (n < 1: the OpenMP default)."""
    lib().oracle_set_threads(int(n))


def max_threads():
    """Threads the next loop over outputs will use."""
    return int(lib().oracle_max_threads())


def half_to_double(bits):
    return lib().oracle_half_to_double(int(bits))


def double_to_half(v):
    return lib().oracle_double_to_half(float(v))


def codebook():
    p = lib().oracle_codebook()
    return np.array([p[i] for i in range(16)], dtype=np.int64)


def quantize_q8_1(x):
    """fp32 [M][K] -> uint8 [M][K/32*36] Q8_1 blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    assert K % 32 == 0
    out = np.empty((M, K // 32 * 36), dtype=np.uint8)
    lib().oracle_quantize_q8_1(_ptr(x), M, K, _ptr(out))
    return out


def rmsnorm(x, w, eps):
    """RMSNorm of each row of fp32 [M][K] with weight w[K] (oracle.c,
    oracle_rmsnorm: Kestrel #18 section 3.6 numerics, 8-element group sums
    added left to right);
    returns (xn fp32 [M][K], ss fp32 [M])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, K = x.shape
    assert K % 32 == 0 and w.shape == (K,)
    xn = np.empty((M, K), dtype=np.float32)
    ss = np.empty(M, dtype=np.float32)
    lib().oracle_rmsnorm(_ptr(x), _ptr(w), float(eps), M, K, _ptr(xn), _ptr(ss))
    return xn, ss


def rmsnorm_quantize_q8_1(x, w, eps):
    """The fused producer's output: Q8_1 blocks of RMSNorm(x) * w."""
    xn, _ = rmsnorm(x, w, eps)
    return quantize_q8_1(xn)


def dequant_q8_1(xq, M, K):
    xq = _u8(xq)
    out = np.empty((M, K), dtype=np.float64)
    lib().oracle_dequant_q8_1(_ptr(xq), M, K, _ptr(out))
    return out


def dequant(W, wtype, N, K):
    W = _u8(W)
    assert W.size == N * (K // 256) * BLOCK_BYTES[wtype]
    out = np.empty((N, K), dtype=np.float64)
    rc = lib().oracle_dequant(_ptr(W), wtype, N, K, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant: bad arguments")
    return out


def isums(W, wtype, N, K, xq, M):
    """int64 [M][N][K/S] exact sub-block dots."""
    W, xq = _u8(W), _u8(xq)
    assert W.size == N * (K // 256) * BLOCK_BYTES[wtype]
    assert xq.size == M * (K // 32) * 36
    out = np.empty((M, N, K // SUBLEN[wtype]), dtype=np.int64)
    rc = lib().oracle_isums(_ptr(W), wtype, N, K, _ptr(xq), M, _ptr(out))
    if rc:
        raise ValueError("oracle_isums: bad arguments")
    return out


def qmatmul(W, wtype, N, K, xq, M):
    """Returns (y64 [M][N] fp64, absum [M][N] fp64, y32 [M][N] fp32)."""
    W, xq = _u8(W), _u8(xq)
    assert W.size == N * (K // 256) * BLOCK_BYTES[wtype]
    assert xq.size == M * (K // 32) * 36
    y64 = np.empty((M, N), dtype=np.float64)
    ab = np.empty((M, N), dtype=np.float64)
    y32 = np.empty((M, N), dtype=np.float32)
    rc = lib().oracle_qmatmul(_ptr(W), wtype, N, K, _ptr(xq), M, _ptr(y64), _ptr(ab), _ptr(y32))
    if rc:
        raise ValueError("oracle_qmatmul: bad arguments")
    return y64, ab, y32


def qmatmul_rows(W, wtype, N, K, xq, M, rows):
    """Selected output columns: returns (y64 [M][len(rows)], absum)."""
    W, xq = _u8(W), _u8(xq)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    y64 = np.empty((M, rows.size), dtype=np.float64)
    ab = np.empty((M, rows.size), dtype=np.float64)
    rc = lib().oracle_qmatmul_rows(_ptr(W), wtype, N, K, _ptr(xq), M, _ptr(rows), rows.size,
                                   _ptr(y64), _ptr(ab))
    if rc:
        raise ValueError("oracle_qmatmul_rows: bad arguments")
    return y64, ab


def kv4_row_bytes(D):
    """Bytes of one K or V row of D elements: D/32 Q4_0 blocks of 18 bytes."""
    return D // 32 * 18


def attn_decode_kv4(q_q8, Hq, Kc, Vc, Hkv, T, D, scale):
    """One decode step of attention over the int4 KV cache (oracle.c,
    oracle_attn_decode_kv4: xLLM v0.7 section C.3, Kestrel #18 online-softmax
    decode).  q_q8: Q8_1 blocks [Hq][D/32]; Kc, Vc: uint8 [Hkv][T][D/32*18].
    Returns (out fp64 [Hq][D], scores fp64 [Hq][T])."""
    q_q8, Kc, Vc = _u8(q_q8), _u8(Kc), _u8(Vc)
    assert q_q8.size == Hq * (D // 32) * 36
    assert Kc.size == Hkv * T * kv4_row_bytes(D) and Vc.size == Kc.size
    out = np.empty((Hq, D), dtype=np.float64)
    sc = np.empty((Hq, T), dtype=np.float64)
    rc = lib().oracle_attn_decode_kv4(_ptr(q_q8), Hq, _ptr(Kc), _ptr(Vc), Hkv, T, D,
                                      float(scale), _ptr(out), _ptr(sc))
    if rc:
        raise ValueError("oracle_attn_decode_kv4: bad arguments")
    return out, sc
