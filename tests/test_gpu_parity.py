"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: Q8_1 bytes bit-exact; integer sub-block sums bit-exact (debug dump);
fp32 y within relative 1e-5 of the oracle's fp64 result on every output;
y fully written (NaN-poisoned before each call); bitwise determinism and
batch invariance (row m of y is identical for every M within one kernel's
range: 1..8 (1..16 for Q4_K and IQ4_XS), then up to 96, above 96).
"""
import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd
from quant_integer_dot_amd import synth

from gpu_util import assert_close, qmatmul, quantize, to_dev

pytestmark = pytest.mark.gpu
TYPES = [synth.Q4_K, synth.Q6_K, synth.IQ4_XS, synth.Q4_0, synth.Q8_0]
TN = synth.TYPE_NAMES


def mid_lo(wtype):
    """Smallest M that runs the mid-batch kernel for this type."""
    return 17 if wtype in (synth.Q4_K, synth.IQ4_XS) else 9


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


# ------------------------------------------------------------- quantizer
@pytest.mark.parametrize("M,K", [(1, 32), (1, 1536), (3, 4096), (8, 12288), (8, 17408),
                                 (5, 8960), (512, 4096), (512, 12288)])
def test_quantizer_bytes_exact(M, K):
    x = synth.activations(M, K, (2026, 77, K, M, 7))
    _, got = quantize(x)
    assert np.array_equal(got, oracle.quantize_q8_1(x).reshape(-1)), (M, K)


def test_quantizer_edge_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 1024)).astype(np.float32)
    x[0, 0:32] = 0.0                                      # amax = 0
    x[1, 32:64] *= np.float32(3e-5)                       # subnormal fp16 d
    x[2, 64:96] = np.float32(127.0)
    x[2, 65:73] = [0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5]  # exact ties
    x[3, 96:128] = -np.abs(x[3, 96:128])                  # all negative
    x[3, 128:160] = np.float32(1e-38)                     # fp32-subnormal-ish inputs
    x[3, 160:192] = np.float32(200.0) * np.sign(x[3, 160:192])
    x[3, 192:224] = -np.abs(x[3, 192:224]) * np.float32(1e-12)  # D = +0, sum(q) < 0: S = -0
    x[3, 224:256] = np.abs(x[3, 224:256]) * np.float32(1e-12)   # D = +0, sum(q) > 0: S = +0
    _, got = quantize(x)
    assert np.array_equal(got, oracle.quantize_q8_1(x).reshape(-1))


def near_half_integer_blocks(nblk, seed):
    """Blocks whose values sit within a few ulps of (k + 1/2) * d32 (d32 the
    block's scale): the quantizer's rounding decisions there depend on the
    correctly rounded quotient, and the reciprocal shortcut must hand them to
    the division.  Also the block of the oracle's division pin."""
    rng = np.random.default_rng(seed)
    x = np.zeros((nblk, 32), np.float32)
    for b in range(nblk):
        A = np.float32(rng.uniform(0.1, 50.0)) * np.float32(2.0 ** int(rng.integers(-20, 20)))
        d32 = np.float32(A / np.float32(127.0))
        x[b, 0] = A if rng.random() < 0.5 else -A
        for i in range(1, 32):
            k = int(rng.integers(-127, 127))
            v = np.float32((k + 0.5) * np.float64(d32))
            for _ in range(int(rng.integers(-3, 4))):
                v = np.nextafter(v, np.float32(np.inf))
            if abs(v) > A:
                v = np.float32(0.0)
            x[b, i] = v
    pin = [1.6125396490097046, 0.08253155648708344, -0.33647480607032776, 0.5269322395324707,
           -0.5396293997764587, 0.0698343887925148, 0.03174290433526039, -0.057137228548526764]
    x[0] = 0.0
    x[0, :len(pin)] = pin
    return x


def test_quantizer_near_half_integers():
    """Byte-exact against the oracle on values at the quantizer's rounding
    boundaries (both the reciprocal path and its division fallback run)."""
    x = near_half_integer_blocks(4096, 5).reshape(8, -1)
    _, got = quantize(x)
    assert np.array_equal(got, oracle.quantize_q8_1(x).reshape(-1))


# ---------------------------------------------------------------- matmul
CASES = [
    # (N, K): several 32-row workgroup tiles plus ragged tails, one superblock
    # up to multi-chunk K
    (1, 256), (37, 256), (100, 512), (257, 1536), (64, 4096), (129, 5120), (50, 8960),
]


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("N,K", CASES)
def test_qmatmul_parity_all_M(wtype, N, K):
    W = synth.weights(wtype, N, K, (2026, 50, N, K + wtype))
    Wd = to_dev(W)
    x = synth.activations(8, K, (2026, 50, K, 8, 7))
    xqd, xq = quantize(x)
    y64_all, _, _ = oracle.qmatmul(W, wtype, N, K, xq, 8)
    is_all = oracle.isums(W, wtype, N, K, xq, 8)
    ref_rows = None
    for M in range(1, 9):
        y, isums = qmatmul(Wd, wtype, N, K, xqd, M, dump=True)
        assert np.array_equal(isums, is_all[:M]), f"{TN[wtype]} N={N} K={K} M={M}: isums differ"
        assert_close(y, y64_all[:M], f"{TN[wtype]} N={N} K={K} M={M}")
        y_plain, _ = qmatmul(Wd, wtype, N, K, xqd, M)
        assert np.array_equal(y_plain.view(np.uint32), y.view(np.uint32)), "dump changes y"
        # batch invariance: rows are bitwise identical for every M
        if ref_rows is None:
            ref_rows = y_plain
        assert np.array_equal(y_plain[:1].view(np.uint32), ref_rows[:1].view(np.uint32))
        if M == 8:
            for Mp in range(1, 8):
                yp, _ = qmatmul(Wd, wtype, N, K, xqd, Mp)
                assert np.array_equal(yp.view(np.uint32), y_plain[:Mp].view(np.uint32)), \
                    f"batch invariance broken at M={Mp}"


@pytest.mark.parametrize("wtype", TYPES)
def test_deterministic(wtype):
    N, K, M = 300, 4096, 8
    W = synth.weights(wtype, N, K, (3, wtype))
    Wd = to_dev(W)
    xqd, _ = quantize(synth.activations(M, K, (4, K, M)))
    y1, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    y2, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("wtype", TYPES)
def test_one_hot_probes_rebuild_dequant(wtype):
    """x = (127/64) e_k gives y[n] = (127/64) w[n, k] exactly: sweeping k
    through every position of two superblocks rebuilds the dequantized
    matrix through the GPU path, pinning every element-to-bit mapping."""
    N, K = 40, 512
    W = synth.weights(wtype, N, K, (5, wtype))
    Wd = to_dev(W)
    wdeq = oracle.dequant(W, wtype, N, K)
    for k0 in range(0, K, 8):
        x = np.zeros((8, K), np.float32)
        for i in range(8):
            x[i, k0 + i] = np.float32(127 * 2.0 ** -6)
        xqd, _ = quantize(x)
        y, _ = qmatmul(Wd, wtype, N, K, xqd, 8)
        exp = (127 / 64) * wdeq[:, k0:k0 + 8].T
        assert np.array_equal(y, exp.astype(np.float32)), f"{TN[wtype]} k0={k0}"


@pytest.mark.parametrize("wtype", TYPES)
def test_one_hot_probes_prefill_path(wtype):
    """The same closed form through the MFMA kernel (M = 40 one-hot rows per
    launch): pins the MFMA operand and result layouts element by element."""
    N, K, M = 70, 512, 40
    W = synth.weights(wtype, N, K, (6, wtype))
    Wd = to_dev(W)
    wdeq = oracle.dequant(W, wtype, N, K)
    for k0 in range(0, K, M):
        x = np.zeros((M, K), np.float32)
        ks = [k0 + i for i in range(M) if k0 + i < K]
        for i, k in enumerate(ks):
            x[i, k] = np.float32(127 * 2.0 ** -6)
        xqd, _ = quantize(x)
        y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
        exp = (127 / 64) * wdeq[:, ks].T
        assert np.array_equal(y[:len(ks)], exp.astype(np.float32)), f"{TN[wtype]} k0={k0}"
        assert not y[len(ks):].any()


@pytest.mark.parametrize("wtype", TYPES)
def test_row_subset(wtype):
    N, K, M = 200, 1536, 3
    W = synth.weights(wtype, N, K, (6, wtype))
    Wd = to_dev(W)
    xqd, _ = quantize(synth.activations(M, K, (7, K, M)))
    y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    n0, n1 = 33, 171
    Wsub = Wd.reshape(-1)[n0 * qd.qdot_weight_bytes(wtype, 1, K):]   # W + n0*row_bytes
    ys, _ = qmatmul(Wsub, wtype, n1 - n0, K, xqd, M)
    assert np.array_equal(ys.view(np.uint32), y[:, n0:n1].view(np.uint32))


def test_zero_activations_give_zero():
    for wtype in TYPES:
        N, K = 64, 1024
        Wd = to_dev(synth.weights(wtype, N, K, (8, wtype)))
        xqd, _ = quantize(np.zeros((4, K), np.float32))
        y, _ = qmatmul(Wd, wtype, N, K, xqd, 4)
        assert not y.any()


def test_q6k_long_rows_all_M():
    """Q6_K rows of 48 and 51 superblocks (the down projection's K = 12288,
    and a K whose superblocks do not divide evenly over the waves of the K
    split): sub-block sums bit-exact through the dump at every M = 1..8, every
    output within 1e-5 rel, and rows bitwise the same at every M."""
    for K in (12288, 13056):
        N = 37
        W = synth.weights(synth.Q6_K, N, K, (2026, 90, K))
        Wd = to_dev(W)
        x = synth.activations(8, K, (2026, 90, K, 8, 7))
        xqd, xq = quantize(x)
        y8, _ = qmatmul(Wd, synth.Q6_K, N, K, xqd, 8)
        y64, _, _ = oracle.qmatmul(W, synth.Q6_K, N, K, xq, 8)
        assert_close(y8, y64, f"Q6_K {N}x{K} M=8")
        for M in range(1, 9):
            xm = xqd[: qd.qdot_q8_1_bytes(M, K)]
            y, isums = qmatmul(Wd, synth.Q6_K, N, K, xm, M, dump=True)
            assert np.array_equal(isums, oracle.isums(W, synth.Q6_K, N, K, xq[: qd.qdot_q8_1_bytes(M, K)], M))
            assert np.array_equal(y.view(np.uint32), y8[:M].view(np.uint32)), f"K={K} M={M}: rows differ from M=8"


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("M", [9, 16, 33, 96, 97, 300])
def test_qmatmul_m_above_8(wtype, M):
    N, K = 70, 1536
    W = synth.weights(wtype, N, K, (9, wtype, M))
    Wd = to_dev(W)
    x = synth.activations(M, K, (10, K, M))
    xqd, xq = quantize(x)
    y, isums = qmatmul(Wd, wtype, N, K, xqd, M, dump=True)
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq, M)
    assert np.array_equal(isums, oracle.isums(W, wtype, N, K, xq, M))
    assert_close(y, y64, f"{TN[wtype]} M={M}")


# ------------------------------ the MFMA decode tile at M = 9..16 (Q4_K, IQ4_XS)
@pytest.mark.parametrize("wtype", [synth.Q4_K, synth.IQ4_XS])
@pytest.mark.parametrize("N,K", [(37, 256), (300, 4608), (129, 5120)])
def test_decode16_rows_and_isums(wtype, N, K):
    """Q4_K and IQ4_XS keep the MFMA decode tile up to M = 16 (16-row A-tile
    slots): sub-block sums bit-exact through the dump at M = 9, 12 and 16,
    every output within 1e-5 rel, and every row bitwise the one of M = 1..8
    (ragged tiles of N, K split unevenly over the waves)."""
    W = synth.weights(wtype, N, K, (2026, 76, wtype, N, K))
    Wd = to_dev(W)
    x = synth.activations(16, K, (2026, 76, K, 16, 7))
    xqd, xq = quantize(x)
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq, 16)
    is_all = oracle.isums(W, wtype, N, K, xq, 16)
    y16, _ = qmatmul(Wd, wtype, N, K, xqd, 16)
    assert_close(y16, y64, f"{TN[wtype]} {N}x{K} M=16")
    for M in range(1, 17):
        assert qd.qdot_kernel_name_shape(wtype, N, K, M).startswith("qmv_")
        xm = xqd[: qd.qdot_q8_1_bytes(M, K)]
        if M in (9, 12, 16):
            y, isums = qmatmul(Wd, wtype, N, K, xm, M, dump=True)
            assert np.array_equal(isums, is_all[:M]), f"M={M}: isums differ"
        else:
            y, _ = qmatmul(Wd, wtype, N, K, xm, M)
        assert np.array_equal(y.view(np.uint32), y16[:M].view(np.uint32)), f"M={M}: rows differ from M=16"


DEC16_FULL = [(name, N, K, t) for (name, N, K, t) in synth.QWEN3_8B + synth.IQ4XS_H5120
              if t in (synth.Q4_K, synth.IQ4_XS)]


@pytest.mark.parametrize("name,N,K,wtype", DEC16_FULL)
def test_decode16_full_size_sampled(name, N, K, wtype):
    """M = 16 on the MFMA decode tile at the full projection shapes: sampled
    rows against the oracle, rows of M = 13 and M = 1 bitwise equal to them."""
    M = 16
    W = synth.weights(wtype, N, K, (2026, 77, N, K))
    Wd = to_dev(W)
    x = synth.activations(M, K, (2026, 77, K, M, 7))
    xqd, xq = quantize(x)
    y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    rng = np.random.default_rng(N + K + 3)
    rows = np.unique(np.concatenate([rng.integers(0, N, 24), [0, N - 1]]))
    y64, _ = oracle.qmatmul_rows(W, wtype, N, K, xq, M, rows)
    assert_close(y[:, rows], y64, f"{name} {N}x{K} M={M}")
    for Mp in (13, 1):
        yp, _ = qmatmul(Wd, wtype, N, K, xqd[: qd.qdot_q8_1_bytes(Mp, K)], Mp)
        assert np.array_equal(yp.view(np.uint32), y[:Mp].view(np.uint32)), f"M={Mp} vs M=16"


# ------------------------------------------------- mid-batch (8 < M <= 96)
@pytest.mark.parametrize("wtype", TYPES)
def test_mid_batch_parity_and_invariance(wtype):
    """M = 9..96 runs the 16-row MFMA kernel with an eight-way K split: sums
    exact, outputs within 1e-5, and every row bitwise the same whatever M of
    that range it is computed in."""
    N, K, M = 300, 2048, 27
    W = synth.weights(wtype, N, K, (2026, 72, wtype))
    Wd = to_dev(W)
    x = synth.activations(96, K, (2026, 72, K, 96, 7))
    xqd, xq = quantize(x)
    row = K // 32 * 36
    y, isums = qmatmul(Wd, wtype, N, K, xqd[:M * row], M, dump=True)
    assert np.array_equal(isums, oracle.isums(W, wtype, N, K, xq[:M * row], M))
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq[:M * row], M)
    assert_close(y, y64, f"{TN[wtype]} M={M}")
    ym96, _ = qmatmul(Wd, wtype, N, K, xqd, 96)
    lo = mid_lo(wtype)
    ylo, _ = qmatmul(Wd, wtype, N, K, xqd, lo)
    assert qd.qdot_kernel_name_shape(wtype, N, K, lo).startswith("qmm_skinny")
    assert np.array_equal(ym96[:M].view(np.uint32), y.view(np.uint32)), "M=96 vs M=27"
    assert np.array_equal(ylo.view(np.uint32), y[:lo].view(np.uint32)), f"M={lo} vs M=27"


@pytest.mark.parametrize("wtype,N,Mlo", [(synth.Q4_K, 2048, 32), (synth.Q6_K, 4096, 16)])
def test_mid_batch_tile_width_invariance(wtype, N, Mlo):
    """Mlo runs one 16-row weight tile per wave, Mlo + 1 two (the grid reaches
    144 workgroups); the shared rows are bitwise equal and both calls match
    the oracle."""
    K, Mhi = 512, Mlo + 1
    W = synth.weights(wtype, N, K, (2026, 73, wtype))
    Wd = to_dev(W)
    x = synth.activations(Mhi, K, (2026, 73, K, Mhi, 7))
    xqd, xq = quantize(x)
    assert qd.qdot_kernel_name_shape(wtype, N, K, Mlo).startswith("qmm_skinny")
    assert qd.qdot_kernel_name_shape(wtype, N, K, Mhi).startswith("qmm_skinny")
    yhi, _ = qmatmul(Wd, wtype, N, K, xqd, Mhi)
    ylo, _ = qmatmul(Wd, wtype, N, K, xqd[: qd.qdot_q8_1_bytes(Mlo, K)], Mlo)
    assert np.array_equal(ylo.view(np.uint32), yhi[:Mlo].view(np.uint32))
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq, Mhi)
    assert_close(yhi, y64, f"{TN[wtype]} N={N} M={Mhi}")


MID_FULL = [(name, N, K, t) for (name, N, K, t) in synth.QWEN3_8B] + \
           [(name, N, K, t) for (name, N, K, t) in synth.IQ4XS_H5120] + \
           [("q4_0-gate", 12288, 4096, synth.Q4_0), ("q8_0-down", 4096, 12288, synth.Q8_0)]


@pytest.mark.parametrize("name,N,K,wtype", MID_FULL)
def test_mid_batch_full_size_sampled(name, N, K, wtype):
    """M = 32 at the full projection shapes: sampled weight rows against the
    oracle, and the rows of a call at the lowest mid-batch M bitwise equal to
    them."""
    M = 32
    W = synth.weights(wtype, N, K, (2026, 74, N, K))
    Wd = to_dev(W)
    x = synth.activations(M, K, (2026, 74, K, M, 7))
    xqd, xq = quantize(x)
    y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    rng = np.random.default_rng(N + K + 2)
    rows = np.unique(np.concatenate([rng.integers(0, N, 24), [0, N - 1]]))
    y64, _ = oracle.qmatmul_rows(W, wtype, N, K, xq, M, rows)
    assert_close(y[:, rows], y64, f"{name} {N}x{K} M={M}")
    lo = mid_lo(wtype)
    ylo, _ = qmatmul(Wd, wtype, N, K, xqd[: qd.qdot_q8_1_bytes(lo, K)], lo)
    assert np.array_equal(ylo.view(np.uint32), y[:lo].view(np.uint32)), "M invariance"


@pytest.mark.parametrize("wtype,N,K,M_switch", [(synth.Q4_K, 8192, 4096, 32), (synth.IQ4_XS, 8192, 4096, 48),
                                                  (synth.Q6_K, 1024, 4096, 256), (synth.Q4_K, 1024, 4096, 128),
                                                  (synth.Q6_K, 4096, 2048, 128)])
def test_matrix_kernel_switch(wtype, N, K, M_switch):
    """The mid-batch kernel's range depends on the matrix (qdot_kernel_name_shape
    says which kernel runs): sampled rows on both sides of the switch against
    the oracle, and rows bitwise equal for every M within each side (the lowest
    mid-batch M vs M_switch, M_switch + 1 vs M_switch + 40)."""
    Mmax = M_switch + 40
    W = synth.weights(wtype, N, K, (2026, 75, wtype, N, K))
    Wd = to_dev(W)
    x = synth.activations(Mmax, K, (2026, 75, K, Mmax, 7))
    xqd, xq = quantize(x)
    assert qd.qdot_kernel_name_shape(wtype, N, K, M_switch).startswith("qmm_skinny")
    assert qd.qdot_kernel_name_shape(wtype, N, K, M_switch + 1).startswith("qmm_mfma")
    rows = np.unique(np.concatenate([np.random.default_rng(N + 5).integers(0, N, 12), [0, N - 1]]))
    ys = {}
    lo = mid_lo(wtype)
    for M in (lo, M_switch, M_switch + 1, Mmax):
        y, _ = qmatmul(Wd, wtype, N, K, xqd[: qd.qdot_q8_1_bytes(M, K)], M)
        y64, _ = oracle.qmatmul_rows(W, wtype, N, K, xq[: qd.qdot_q8_1_bytes(M, K)], M, rows)
        assert_close(y[:, rows], y64, f"{TN[wtype]} {N}x{K} M={M}")
        ys[M] = y
    assert np.array_equal(ys[lo].view(np.uint32), ys[M_switch][:lo].view(np.uint32)), "mid-batch rows"
    s1 = M_switch + 1
    assert np.array_equal(ys[s1].view(np.uint32), ys[Mmax][:s1].view(np.uint32)), "prefill rows"


# --------------------------------------------------- prefill (MFMA path)
@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("M,N,K", [(512, 200, 768), (300, 64, 256), (260, 333, 1280), (130, 4096, 512)])
def test_prefill_parity(wtype, M, N, K):
    """Several 128 x 64 output tiles with ragged edges in M and N: sub-block
    sums bit-exact through the dump, every output within 1e-5 rel."""
    W = synth.weights(wtype, N, K, (2026, 70, wtype, N, K))
    Wd = to_dev(W)
    x = synth.activations(M, K, (2026, 70, K, M, 7))
    xqd, xq = quantize(x)
    y, isums = qmatmul(Wd, wtype, N, K, xqd, M, dump=True)
    assert np.array_equal(isums, oracle.isums(W, wtype, N, K, xq, M))
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq, M)
    assert_close(y, y64, f"{TN[wtype]} M={M} {N}x{K}")
    y2, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    assert np.array_equal(y2.view(np.uint32), y.view(np.uint32)), "dump changed y"


PREFILL = [(name, N, K, t) for (name, N, K, t) in synth.QWEN3_8B]


@pytest.mark.parametrize("name,N,K,wtype", PREFILL)
def test_prefill_full_size_sampled(name, N, K, wtype):
    """M=512 at the 8B projection shapes, in the launch the benchmark times;
    256 seeded weight rows (plus the first and last) against the oracle, and
    rows of a smaller M > 8 call bitwise equal to the same rows of the M=512
    call."""
    M = 512
    W = synth.weights(wtype, N, K, (2026, 71, N, K))
    Wd = to_dev(W)
    x = synth.activations(M, K, (2026, 71, K, M, 7))
    xqd, xq = quantize(x)
    y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    rng = np.random.default_rng(N + K + 1)
    rows = np.unique(np.concatenate([rng.choice(N, 256, replace=False), [0, N - 1]]))
    assert rows.size >= 256
    y64, _ = oracle.qmatmul_rows(W, wtype, N, K, xq, M, rows)
    assert_close(y[:, rows], y64, f"{name} {N}x{K} M=512")
    Ms = 300  # above every matrix's mid-batch range, so the same kernel
    y_s, _ = qmatmul(Wd, wtype, N, K, xqd[: qd.qdot_q8_1_bytes(Ms, K)], Ms)
    assert np.array_equal(y_s.view(np.uint32), y[:Ms].view(np.uint32)), "M invariance"


# ------------------------------------------- full-size shapes, sampled rows
FULL = [(name, N, K, t) for (name, N, K, t) in synth.QWEN3_8B] + \
       [(name, N, K, t) for (name, N, K, t) in synth.IQ4XS_H5120] + \
       [("c1-down", 1536, 8960, synth.Q4_K), ("c0", 1536, 1536, synth.Q4_K),
        ("q4_0-gate", 12288, 4096, synth.Q4_0), ("q8_0-down", 4096, 12288, synth.Q8_0)]


@pytest.mark.parametrize("name,N,K,wtype", FULL)
def test_full_size_all_rows(name, N, K, wtype):
    """M = 8 at the full projection shapes (the Qwen3-8B and hidden-5120
    matrices, Qwen2.5-1.5B's down, the single 1536 x 1536 matrix, the Q4_0 /
    Q8_0 variants): every output against the oracle; rows of M = 1 bitwise
    equal to those of M = 8."""
    M = 8
    W = synth.weights(wtype, N, K, (2026, 60, N, K))
    Wd = to_dev(W)
    x = synth.activations(M, K, (2026, 60, K, M, 7))
    xqd, xq = quantize(x)
    y, _ = qmatmul(Wd, wtype, N, K, xqd, M)
    y64, _, _ = oracle.qmatmul(W, wtype, N, K, xq, M)
    assert_close(y, y64, f"{name} {N}x{K}")
    y1, _ = qmatmul(Wd, wtype, N, K, xqd, 1)
    assert np.array_equal(y1.view(np.uint32), y[:1].view(np.uint32)), "batch invariance"


# ------------------------------------- negative fp16 scales, every kernel
@pytest.mark.parametrize("wtype", TYPES)
def test_signed_scales_every_kernel(wtype):
    """Weights whose fp16 d (and Q4_K dmin) carry random signs, through the
    decode tiles (M = 1..8; for Q4_K and IQ4_XS the 16-row tile at M = 12),
    the mid-batch kernel (M = 40) and the prefill kernel (M = 300): sub-block
    sums exact through the dump, every output within 1e-5 rel."""
    N, K = 133, 2560
    W = synth.weights(wtype, N, K, (2026, 78, wtype), signed_scales=True)
    d = W.reshape(N, K // 256, -1)
    d16 = d[:, :, 0:2].copy().view(np.float16)[..., 0] if wtype not in (synth.Q6_K,) else \
        d[:, :, 208:210].copy().view(np.float16)[..., 0]
    assert (d16 < 0).any() and (d16 > 0).any()
    Wd = to_dev(W)
    x = synth.activations(300, K, (2026, 78, K, 300, 7))
    xqd, xq = quantize(x)
    for M in (1, 2, 3, 5, 8, 12, 40, 300):
        xm, xmh = xqd[: qd.qdot_q8_1_bytes(M, K)], xq[: qd.qdot_q8_1_bytes(M, K)]
        y, isums = qmatmul(Wd, wtype, N, K, xm, M, dump=M in (1, 8, 12, 40, 300))
        y64, _, _ = oracle.qmatmul(W, wtype, N, K, xmh, M)
        assert_close(y, y64, f"{TN[wtype]} signed scales M={M}")
        if isums is not None:
            assert np.array_equal(isums, oracle.isums(W, wtype, N, K, xmh, M)), f"M={M}: isums differ"


# ------------------------------------------------- the pages' noise anchor
def test_noise_against_fp32_sgemv():
    """About 0.5 % RMS against unquantized fp32 SGEMV, argmax kept (xLLM B1.3)."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "q8_activation_noise.json")))
    N, K, M = 2048, 4096, 4
    for wtype in TYPES:
        W = synth.weights(wtype, N, K, (2026, 61, wtype, 0))
        x = synth.activations(M, K, (2026, 61, K, M, 7))
        xqd, _ = quantize(x)
        y, _ = qmatmul(to_dev(W), wtype, N, K, xqd, M)
        ref = (x @ oracle.dequant(W, wtype, N, K).astype(np.float32).T).astype(np.float64)
        rel = np.sqrt(np.mean((y - ref) ** 2) / np.mean(ref ** 2))
        lo, hi = g["test_band"]
        assert lo <= rel <= hi, (TN[wtype], rel)
        for m in range(M):
            top = np.argsort(ref[m])[::-1]
            if ref[m, top[0]] - ref[m, top[1]] > 6 * rel * np.sqrt(np.mean(ref[m] ** 2)):
                assert int(np.argmax(y[m])) == int(top[0])
