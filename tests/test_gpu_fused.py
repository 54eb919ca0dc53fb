"""GPU: the activation quantizer fused into the decode matmul
(qdot_quantize_qmatmul, qdot_quantize_qmatmul_multi).  The kernel quantizes
with the standalone quantizer's own device code, so y must be bitwise the y
of qdot_quantize_q8_1 followed by qdot_qmatmul (or qdot_qmatmul_multi); every
output is also checked against the oracle (quantizer and matmul)."""
import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd
from quant_integer_dot_amd import synth

from gpu_util import assert_close, dev, qmatmul, quantize, to_dev
from test_gpu_parity import near_half_integer_blocks

pytestmark = pytest.mark.gpu
TYPES = [synth.Q4_K, synth.Q6_K, synth.IQ4_XS, synth.Q4_0, synth.Q8_0]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


def fused(Wd, wtype, N, K, x_h, M):
    import torch
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
    qd.qdot_quantize_qmatmul(Wd, wtype, N, K, to_dev(x_h[:M].astype(np.float32)), M, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("N,K", [(37, 256), (257, 1536), (129, 5120), (64, 12288)])
def test_fused_equals_quantize_then_qmatmul(wtype, N, K):
    W = synth.weights(wtype, N, K, (2026, 81, wtype, N, K))
    Wd = to_dev(W)
    x = synth.activations(8, K, (2026, 81, K, 8, 7))
    x[0, 32:64] = 0.0                      # an all-zero block (amax = 0)
    x[1, 64:96] *= np.float32(1e-6)        # a subnormal fp16 d
    for M in range(1, 9):
        xqd, xq = quantize(x[:M])
        y_ref, _ = qmatmul(Wd, wtype, N, K, xqd, M)
        y = fused(Wd, wtype, N, K, x, M)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), f"{wtype} {N}x{K} M={M}"
        if M in (1, 2, 8):
            y64, _, _ = oracle.qmatmul(W, wtype, N, K, oracle.quantize_q8_1(x[:M]), M)
            assert_close(y, y64, f"fused {wtype} {N}x{K} M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 8])
def test_fused_groups_headline_shapes(M):
    """q+k+v (Q4_K, Q4_K, Q6_K) and gate+up (two Q4_K) of the 8B model at full
    size: each matrix bitwise equal to quantize + qdot_qmatmul_multi (which
    may run MFMA tiles: their rows are bitwise the dot4 tile's), and every
    output against the oracle."""
    import torch
    K = 4096
    x = synth.activations(M, K, (2026, 82, K, M, 7))
    xd = to_dev(x)
    xqd, xq = quantize(x)
    for mats, seed in (([(4096, synth.Q4_K), (1024, synth.Q4_K), (1024, synth.Q6_K)], 1),
                       ([(12288, synth.Q4_K), (12288, synth.Q4_K)], 2)):
        Ws = [synth.weights(t, N, K, (2026, 82, seed, i)) for i, (N, t) in enumerate(mats)]
        Wds = [to_dev(W) for W in Ws]
        types, Ns = [t for _, t in mats], [N for N, _ in mats]
        ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev()) for N in Ns]
        yr = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev()) for N in Ns]
        qd.qdot_quantize_qmatmul_multi(Wds, types, Ns, K, xd, M, ys)
        qd.qdot_qmatmul_multi(Wds, types, Ns, K, xqd, M, yr)
        torch.cuda.synchronize()
        for i, (N, t) in enumerate(mats):
            a, b = ys[i].cpu().numpy(), yr[i].cpu().numpy()
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"group {seed} matrix {i} M={M}"
            y64, _, _ = oracle.qmatmul(Ws[i], t, N, K, xq, M)
            assert_close(a, y64, f"fused group {seed} matrix {i} M={M}")


def test_fused_mixed_types_split_launches():
    """IQ4_XS with Q4_K and Q8_0 (one launch per type) through the fused call."""
    import torch
    K, M = 512, 3
    mats = [(48, synth.IQ4_XS), (40, synth.Q4_K), (24, synth.Q8_0), (16, synth.IQ4_XS)]
    x = synth.activations(M, K, (2026, 83, K, M, 7))
    xqd, _ = quantize(x)
    Ws = [to_dev(synth.weights(t, N, K, (2026, 83, i))) for i, (N, t) in enumerate(mats)]
    types, Ns = [t for _, t in mats], [N for N, _ in mats]
    ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev()) for N in Ns]
    qd.qdot_quantize_qmatmul_multi(Ws, types, Ns, K, to_dev(x), M, ys)
    torch.cuda.synchronize()
    for i, (N, t) in enumerate(mats):
        y1, _ = qmatmul(Ws[i], t, N, K, xqd, M)
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), y1.view(np.uint32)), i


@pytest.mark.parametrize("wtype", [synth.Q4_K, synth.Q6_K, synth.Q4_0])
def test_fused_near_half_integers(wtype):
    """Activations at the quantizer's rounding boundaries through the fused
    call: bitwise the standalone quantizer + matmul, sums exact."""
    N, K = 96, 2048
    W = synth.weights(wtype, N, K, (2026, 84, wtype))
    Wd = to_dev(W)
    x = near_half_integer_blocks(2 * K // 32, 11).reshape(2, K)
    for M in (1, 2):
        xqd, xq = quantize(x[:M])
        assert np.array_equal(xq, oracle.quantize_q8_1(x[:M]).reshape(-1))
        y_ref, _ = qmatmul(Wd, wtype, N, K, xqd, M)
        y = fused(Wd, wtype, N, K, x, M)
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), f"M={M}"
