"""C ABI checks that need no GPU: the library loads, exports every function
include/qdot.h declares, computes sizes, and rejects bad arguments before any
HIP call (so nothing is launched and no device is touched)."""
import ctypes
import os
import re

import pytest

from quant_integer_dot_amd import binding as qd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qdot.h")


@pytest.fixture(scope="module")
def lib():
    return qd.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdot_\w+)\s*\(", text)))


def test_header_symbols_exported(lib):
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"libqdot.so does not export {n}"


def test_sizes(lib):
    assert qd.qdot_block_bytes(qd.QDOT_Q4_K) == 144
    assert qd.qdot_block_bytes(qd.QDOT_Q6_K) == 210
    assert qd.qdot_block_bytes(qd.QDOT_IQ4_XS) == 136
    assert qd.qdot_block_bytes(qd.QDOT_Q4_0) == 8 * 18
    assert qd.qdot_block_bytes(qd.QDOT_Q8_0) == 8 * 34
    assert qd.qdot_block_bytes(0) == 0 and qd.qdot_block_bytes(6) == 0
    assert qd.qdot_weight_bytes(qd.QDOT_Q8_0, 4096, 12288) == 4096 * 384 * 34
    assert qd.qdot_isum_count(qd.QDOT_Q4_0, 3, 512, 2) == 2 * 3 * 16
    assert qd.qdot_weight_bytes(qd.QDOT_Q4_K, 12288, 4096) == 12288 * 16 * 144
    assert qd.qdot_weight_bytes(qd.QDOT_Q6_K, 4096, 12288) == 4096 * 48 * 210
    assert qd.qdot_weight_bytes(qd.QDOT_Q4_K, 10, 100) == 0
    assert qd.qdot_q8_1_bytes(8, 17408) == 156672
    assert qd.qdot_q8_1_bytes(1, 33) == 0
    assert qd.qdot_isum_count(qd.QDOT_Q6_K, 3, 512, 2) == 2 * 3 * 32
    assert qd.qdot_isum_count(qd.QDOT_Q4_K, 3, 512, 2) == 2 * 3 * 16


def test_names_and_status(lib):
    assert qd.qdot_kernel_name(qd.QDOT_Q4_K, 8) == "qmv_mfma<Q4_K,8>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_K, 6) == "qmv_dot4<Q4_K,6>"
    assert qd.qdot_kernel_name(qd.QDOT_Q6_K, 8) == "qmv_mfma<Q6_K,8>"
    assert qd.qdot_kernel_name(qd.QDOT_Q6_K, 7) == "qmv_mfma<Q6_K,7>"
    assert qd.qdot_kernel_name(qd.QDOT_Q6_K, 6) == "qmv_dot4<Q6_K,6>"
    assert qd.qdot_kernel_name(qd.QDOT_IQ4_XS, 5) == "qmv_mfma<IQ4_XS,5>"
    assert qd.qdot_kernel_name(qd.QDOT_IQ4_XS, 4) == "qmv_dot4<IQ4_XS,4>"
    assert qd.qdot_kernel_name(qd.QDOT_IQ4_XS, 1) == "qmv_dot4<IQ4_XS,1>"
    assert qd.qdot_kernel_name(qd.QDOT_Q8_0, 4) == "qmv_dot4<Q8_0,4>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_0, 100) == "qmm_mfma<Q4_0>"
    assert qd.qdot_kernel_name(qd.QDOT_Q8_0, 16) == "qmm_skinny<Q8_0>"
    assert qd.qdot_kernel_name(qd.QDOT_Q6_K, 512) == "qmm_mfma<Q6_K>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_K, 9) == "qmv_mfma<Q4_K,9>"
    assert qd.qdot_kernel_name(qd.QDOT_IQ4_XS, 16) == "qmv_mfma<IQ4_XS,16>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_K, 17) == "qmm_skinny<Q4_K>"
    assert qd.qdot_kernel_name(qd.QDOT_Q6_K, 9) == "qmm_skinny<Q6_K>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_0, 9) == "qmm_skinny<Q4_0>"
    assert qd.qdot_kernel_name(qd.QDOT_IQ4_XS, 96) == "qmm_skinny<IQ4_XS>"
    assert qd.qdot_kernel_name(qd.QDOT_Q4_K, 97) == "qmm_mfma<Q4_K>"
    assert qd.qdot_kernel_name(9, 1) == "invalid"
    # the shape-aware name: wide Q4_K / IQ4_XS matrices leave the mid-batch
    # kernel earlier; everything else matches qdot_kernel_name
    ks = qd.qdot_kernel_name_shape
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 32) == "qmm_skinny<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 33) == "qmm_mfma<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 8192, 4096, 33) == "qmm_mfma<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 8191, 4096, 33) == "qmm_skinny<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 12288, 3840, 33) == "qmm_skinny<Q4_K>"
    assert ks(qd.QDOT_IQ4_XS, 17408, 5120, 48) == "qmm_skinny<IQ4_XS>"
    assert ks(qd.QDOT_IQ4_XS, 17408, 5120, 49) == "qmm_mfma<IQ4_XS>"
    assert ks(qd.QDOT_Q6_K, 12288, 4096, 128) == "qmm_skinny<Q6_K>"
    assert ks(qd.QDOT_Q6_K, 12288, 4096, 129) == "qmm_mfma<Q6_K>"
    assert ks(qd.QDOT_Q6_K, 2048, 4096, 256) == "qmm_skinny<Q6_K>"
    assert ks(qd.QDOT_Q6_K, 2048, 4096, 257) == "qmm_mfma<Q6_K>"
    assert ks(qd.QDOT_Q6_K, 2049, 4096, 129) == "qmm_mfma<Q6_K>"
    assert ks(qd.QDOT_Q4_K, 2048, 4096, 128) == "qmm_skinny<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 2048, 4096, 129) == "qmm_mfma<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 4096, 4096, 97) == "qmm_mfma<Q4_K>"
    assert ks(qd.QDOT_Q4_0, 12288, 4096, 96) == "qmm_skinny<Q4_0>"
    assert ks(qd.QDOT_Q4_0, 1024, 4096, 97) == "qmm_mfma<Q4_0>"
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 8) == "qmv_mfma<Q4_K,8>"
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 16) == "qmv_mfma<Q4_K,16>"
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 17) == "qmm_skinny<Q4_K>"
    assert ks(qd.QDOT_IQ4_XS, 17408, 5120, 13) == "qmv_mfma<IQ4_XS,13>"
    assert ks(qd.QDOT_Q6_K, 12288, 4096, 9) == "qmm_skinny<Q6_K>"
    assert ks(qd.QDOT_Q4_K, 12288, 4096, 97) == "qmm_mfma<Q4_K>"
    assert ks(qd.QDOT_Q4_K, 12288, 100, 40) == "invalid"
    for t in (qd.QDOT_Q4_K, qd.QDOT_IQ4_XS, qd.QDOT_Q4_0, qd.QDOT_Q8_0):
        for M in (1, 5, 8, 9, 16, 17, 33, 49, 96, 97, 512):
            assert ks(t, 4096, 4096, M) == qd.qdot_kernel_name(t, M)
    for M in (1, 5, 8, 9, 96, 512):
        assert ks(qd.QDOT_Q6_K, 4096, 4096, M) == qd.qdot_kernel_name(qd.QDOT_Q6_K, M)
    # grouped launches choose the tile per launch: q+k+v of the 8B model
    # (under 4 MB per stage) takes MFMA tiles for its Q4_K matrices at every M,
    # gate+up from M = 3, and at K = 1536 the dot4 tile stays
    mk = qd.qdot_multi_kernel_name
    qkv = ([qd.QDOT_Q4_K, qd.QDOT_Q4_K, qd.QDOT_Q6_K], [4096, 1024, 1024])
    assert [mk(*qkv, 4096, 1, i) for i in range(3)] == ["qmv_mfma<Q4_K,1>", "qmv_mfma<Q4_K,1>", "qmv_dot4<Q6_K,1>"]
    gu = ([qd.QDOT_Q4_K, qd.QDOT_Q4_K], [12288, 12288])
    assert mk(*gu, 4096, 2, 0) == "qmv_dot4<Q4_K,2>"
    assert mk(*gu, 4096, 3, 1) == "qmv_mfma<Q4_K,3>"
    assert mk(*([qd.QDOT_Q4_K, qd.QDOT_Q4_K], [8960, 8960]), 1536, 8, 0) == "qmv_dot4<Q4_K,8>"
    assert mk(*([qd.QDOT_IQ4_XS] * 2, [17408, 17408]), 5120, 4, 0) == "qmv_mfma<IQ4_XS,4>"
    assert mk(*gu, 4096, 64, 0) == "qmm_mfma<Q4_K>"
    assert mk(*gu, 4096, 12, 1) == "qmv_mfma<Q4_K,12>"
    assert mk(*gu, 4096, 17, 1) == "qmm_skinny<Q4_K>"
    assert mk(*gu, 4096, 1, 2) == "invalid"
    assert mk(*([qd.QDOT_Q4_K, 9], [64, 64]), 4096, 1, 0) == "invalid"
    assert qd.qdot_status_str(qd.QDOT_E_ALIGN) == "misaligned pointer"
    assert "gfx950" in qd.qdot_build_id()


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,status", [
    ((FAKE, 7, 16, 256, FAKE, 1, FAKE), qd.QDOT_E_ARG),        # unknown type
    ((FAKE, 1, 0, 256, FAKE, 1, FAKE), qd.QDOT_E_ARG),         # N < 1
    ((FAKE, 1, 16, 255, FAKE, 1, FAKE), qd.QDOT_E_ARG),        # K % 256
    ((FAKE, 1, 16, 0, FAKE, 1, FAKE), qd.QDOT_E_ARG),          # K = 0
    ((FAKE, 1, 16, 256, FAKE, 0, FAKE), qd.QDOT_E_ARG),        # M < 1
    ((0, 1, 16, 256, FAKE, 1, FAKE), qd.QDOT_E_ARG),           # null W
    ((FAKE, 1, 16, 256, 0, 1, FAKE), qd.QDOT_E_ARG),           # null x_q8
    ((FAKE, 1, 16, 256, FAKE, 1, 0), qd.QDOT_E_ARG),           # null y
    ((FAKE, 1, 16, 256, FAKE + 2, 1, FAKE), qd.QDOT_E_ALIGN),  # x_q8 misaligned
    ((FAKE, 1, 16, 256, FAKE, 1, FAKE + 1), qd.QDOT_E_ALIGN),  # y misaligned
    ((FAKE, 1, 2**31, 256, FAKE, 1, FAKE), qd.QDOT_E_ARG),     # N too large
])
def test_qmatmul_validation(lib, args, status):
    W, t, N, K, X, M, Y = args
    assert lib.qdot_qmatmul(W, t, N, K, X, M, Y, None) == status
    assert lib.qdot_qmatmul_dump_isums(W, t, N, K, X, M, Y, FAKE, None) == status


def test_dump_needs_isums(lib):
    assert lib.qdot_qmatmul_dump_isums(FAKE, 1, 16, 256, FAKE, 1, FAKE, 0, None) == qd.QDOT_E_ARG
    assert lib.qdot_qmatmul_dump_isums(FAKE, 1, 16, 256, FAKE, 1, FAKE, FAKE + 2, None) == qd.QDOT_E_ALIGN


@pytest.mark.parametrize("args,status", [
    ((0, 1, 32, FAKE), qd.QDOT_E_ARG),
    ((FAKE, 1, 32, 0), qd.QDOT_E_ARG),
    ((FAKE, 0, 32, FAKE), qd.QDOT_E_ARG),
    ((FAKE, 1, 48, FAKE), qd.QDOT_E_ARG),
    ((FAKE + 2, 1, 32, FAKE), qd.QDOT_E_ALIGN),
    ((FAKE, 1, 32, FAKE + 1), qd.QDOT_E_ALIGN),
])
def test_quantize_validation(lib, args, status):
    x, M, K, xq = args
    assert lib.qdot_quantize_q8_1(x, M, K, xq, None) == status


def test_binding_raises_on_error(lib):
    with pytest.raises(qd.QdotError):
        qd.qdot_qmatmul(FAKE, 7, 16, 256, FAKE, 1, FAKE, stream=0)


def test_product_path_does_not_import_oracle():
    """The HIP path never imports or loads the oracle (test infrastructure)."""
    pkg = os.path.join(ROOT, "quant_integer_dot_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "liboracle" not in txt, f


def _multi(lib, n, Ws, types, Ns, K, xq, M, ys):
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    m = max(len(Ws), 1)
    return lib.qdot_qmatmul_multi(n, (P * m)(*Ws), (i32 * m)(*types), (i64 * m)(*Ns), K, xq, M,
                                  (P * m)(*ys), None)


@pytest.mark.parametrize("case,status", [
    (dict(n=0), qd.QDOT_E_ARG),
    (dict(n=5, Ws=[16] * 5, types=[1] * 5, Ns=[16] * 5, ys=[16] * 5), qd.QDOT_E_ARG),
    (dict(K=100), qd.QDOT_E_ARG),
    (dict(types=[1, 9]), qd.QDOT_E_ARG),
    (dict(Ns=[16, 0]), qd.QDOT_E_ARG),
    (dict(M=0), qd.QDOT_E_ARG),
    (dict(Ws=[16, 0]), qd.QDOT_E_ARG),
    (dict(ys=[16, 0]), qd.QDOT_E_ARG),
    (dict(xq=0), qd.QDOT_E_ARG),
    (dict(xq=18), qd.QDOT_E_ALIGN),
    (dict(ys=[16, 34]), qd.QDOT_E_ALIGN),
])
def test_qmatmul_multi_validation(lib, case, status):
    """Every argument of the grouped call is checked before anything is launched."""
    a = dict(n=2, Ws=[16, 16], types=[1, 2], Ns=[16, 16], K=256, xq=16, M=1, ys=[16, 16])
    a.update(case)
    assert _multi(lib, a["n"], a["Ws"], a["types"], a["Ns"], a["K"], a["xq"], a["M"], a["ys"]) == status


def test_binding_multi_lengths(lib):
    with pytest.raises(ValueError):
        qd.qdot_qmatmul_multi([16, 16], [1], [16, 16], 256, 16, 1, [16, 16], stream=0)


@pytest.mark.parametrize("args,status", [
    ((0, 16, 1e-6, 1, 256, 16), qd.QDOT_E_ARG),
    ((16, 0, 1e-6, 1, 256, 16), qd.QDOT_E_ARG),
    ((16, 16, 1e-6, 1, 256, 0), qd.QDOT_E_ARG),
    ((16, 16, 1e-6, 0, 256, 16), qd.QDOT_E_ARG),
    ((16, 16, 1e-6, 1, 100, 16), qd.QDOT_E_ARG),
    ((16, 16, 1e-6, 1, 65536, 16), qd.QDOT_E_ARG),
    ((16, 16, -1.0, 1, 256, 16), qd.QDOT_E_ARG),
    ((16, 16, float("nan"), 1, 256, 16), qd.QDOT_E_ARG),
    ((18, 16, 1e-6, 1, 256, 16), qd.QDOT_E_ALIGN),
    ((16, 16, 1e-6, 1, 256, 18), qd.QDOT_E_ALIGN),
])
def test_rmsnorm_quantize_validation(lib, args, status):
    x, w, eps, M, K, xq = args
    assert lib.qdot_rmsnorm_quantize_q8_1(x, w, eps, M, K, xq, None) == status


def test_attn_sizes(lib):
    assert qd.qdot_attn_kv4_row_bytes(128) == 72
    assert qd.qdot_attn_kv4_row_bytes(64) == 36
    assert qd.qdot_attn_kv4_row_bytes(100) == 0 and qd.qdot_attn_kv4_row_bytes(256) == 0
    # per head and 256-token chunk: max, sum and 128 partial outputs (fp32)
    assert qd.qdot_attn_kv4_workspace_bytes(32, 32768) == 32 * 128 * 130 * 4
    assert qd.qdot_attn_kv4_workspace_bytes(4, 257) == 4 * 2 * 130 * 4
    assert qd.qdot_attn_kv4_workspace_bytes(4, 0) == 0 and qd.qdot_attn_kv4_workspace_bytes(0, 8) == 0


WS = 1 << 20


@pytest.mark.parametrize("args,status", [
    ((0, 32, FAKE, FAKE, 8, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ARG),        # null query
    ((FAKE, 32, FAKE, FAKE, 8, 100, 128, 0.1, FAKE, 0, WS), qd.QDOT_E_ARG),        # null workspace
    ((FAKE, 32, FAKE, FAKE, 8, 100, 64, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ARG),      # D != 128
    ((FAKE, 30, FAKE, FAKE, 8, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ARG),     # Hq % Hkv
    ((FAKE, 32, FAKE, FAKE, 2, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ARG),     # group of 16
    ((FAKE, 32, FAKE, FAKE, 8, 0, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ARG),       # T = 0
    ((FAKE, 32, FAKE, FAKE, 8, 2**26 + 1, 128, 0.1, FAKE, FAKE, 2**40), qd.QDOT_E_ARG),  # T too large
    ((FAKE, 32, FAKE, FAKE, 8, 100, 128, float("nan"), FAKE, FAKE, WS), qd.QDOT_E_ARG),  # NaN scale
    ((FAKE, 32, FAKE, FAKE, 8, 100, 128, float("inf"), FAKE, FAKE, WS), qd.QDOT_E_ARG),  # inf scale
    ((FAKE, 32, FAKE, FAKE, 8, 300, 128, 0.1, FAKE, FAKE, 32 * 2 * 130 * 4 - 4), qd.QDOT_E_ARG),  # short ws
    ((FAKE, 32, FAKE + 4, FAKE, 8, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ALIGN),  # K not 8-aligned
    ((FAKE, 32, FAKE, FAKE + 4, 8, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ALIGN),  # V not 8-aligned
    ((FAKE + 2, 32, FAKE, FAKE, 8, 100, 128, 0.1, FAKE, FAKE, WS), qd.QDOT_E_ALIGN),  # query
    ((FAKE, 32, FAKE, FAKE, 8, 100, 128, 0.1, FAKE + 1, FAKE, WS), qd.QDOT_E_ALIGN),  # out
])
def test_attn_validation(lib, args, status):
    q, Hq, K, V, Hkv, T, D, scale, out, ws, wsb = args
    assert lib.qdot_attn_decode_kv4(q, Hq, K, V, Hkv, T, D, ctypes.c_float(scale), out, ws, wsb, None) == status


@pytest.mark.parametrize("src,nbytes,sink,status", [
    (0, 4096, FAKE, qd.QDOT_E_ARG),            # null source
    (FAKE, 4096, 0, qd.QDOT_E_ARG),            # null sink
    (FAKE, 0, FAKE, qd.QDOT_E_ARG),            # nothing to read
    (FAKE, 4100, FAKE, qd.QDOT_E_ARG),         # not a multiple of 16 bytes
    (FAKE + 8, 4096, FAKE, qd.QDOT_E_ALIGN),   # source not 16-byte aligned
    (FAKE, 4096, FAKE + 2, qd.QDOT_E_ALIGN),   # sink misaligned
])
def test_stream_read_validation(lib, src, nbytes, sink, status):
    assert lib.qdot_stream_read(src, nbytes, sink, None) == status


def test_attn_noalloc_validation(lib):
    """The no-allocation attention call rejects a context whose workspace
    would not fit the static array, and bad arguments, before any HIP call."""
    D = 128
    per_chunk = 4 * (D + 2) * 4                       # Hq = 4
    T_ok = qd.QDOT_ATTN_NOALLOC_BYTES // per_chunk * 256
    assert qd.qdot_attn_kv4_workspace_bytes(4, T_ok) <= qd.QDOT_ATTN_NOALLOC_BYTES
    f = lib.qdot_attn_decode_kv4_noalloc
    assert f(FAKE, 4, FAKE, FAKE, 1, T_ok + 256, D, ctypes.c_float(0.1), FAKE, None) == qd.QDOT_E_ARG
    assert f(0, 4, FAKE, FAKE, 1, 100, D, ctypes.c_float(0.1), FAKE, None) == qd.QDOT_E_ARG
    assert f(FAKE, 4, FAKE, FAKE, 1, 100, 64, ctypes.c_float(0.1), FAKE, None) == qd.QDOT_E_ARG
    assert f(FAKE, 4, FAKE, FAKE, 3, 100, D, ctypes.c_float(0.1), FAKE, None) == qd.QDOT_E_ARG
    assert f(FAKE, 4, FAKE + 4, FAKE, 1, 100, D, ctypes.c_float(0.1), FAKE, None) == qd.QDOT_E_ALIGN
    assert f(FAKE, 4, FAKE, FAKE, 1, 100, D, ctypes.c_float(float("nan")), FAKE, None) == qd.QDOT_E_ARG


def test_quantize_qmatmul_validation(lib):
    """The fused quantizer + matmul calls take M <= 8 and check everything
    before any HIP call."""
    f = lib.qdot_quantize_qmatmul
    assert f(FAKE, 1, 16, 256, FAKE, 9, FAKE, None) == qd.QDOT_E_ARG          # M above the decode range
    assert f(FAKE, 1, 16, 256, FAKE, 0, FAKE, None) == qd.QDOT_E_ARG
    assert f(FAKE, 7, 16, 256, FAKE, 1, FAKE, None) == qd.QDOT_E_ARG          # type
    assert f(FAKE, 1, 16, 300, FAKE, 1, FAKE, None) == qd.QDOT_E_ARG          # K % 256
    assert f(0, 1, 16, 256, FAKE, 1, FAKE, None) == qd.QDOT_E_ARG
    assert f(FAKE, 1, 16, 256, FAKE + 2, 1, FAKE, None) == qd.QDOT_E_ALIGN    # x misaligned
    assert f(FAKE, 1, 16, 256, FAKE, 1, FAKE + 1, None) == qd.QDOT_E_ALIGN
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    w = (P * 2)(FAKE, FAKE)
    t = (i32 * 2)(1, 2)
    n = (i64 * 2)(16, 16)
    y = (P * 2)(FAKE, FAKE)
    g = lib.qdot_quantize_qmatmul_multi
    assert g(2, w, t, n, 256, FAKE, 9, y, None) == qd.QDOT_E_ARG
    assert g(5, w, t, n, 256, FAKE, 1, y, None) == qd.QDOT_E_ARG
    assert g(2, w, t, n, 256, FAKE + 2, 1, y, None) == qd.QDOT_E_ALIGN
