"""GPU: the fused RMSNorm + Q8_1 producer (qdot_rmsnorm_quantize_q8_1)
against the oracle, byte for byte.  The oracle is the Kestrel_VLLM #18
(section 3.6) serial CPU order: 8-element group sums added left to right in
one fp32 accumulator.  The kernel forms the group sums in parallel and adds
them in that order, so every quantized code, D and S must agree exactly."""
import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd

from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


def run(x, w, eps):
    import torch
    M, K = x.shape
    xq = torch.full((qd.qdot_q8_1_bytes(M, K),), 0xA5, dtype=torch.uint8, device=dev())
    qd.qdot_rmsnorm_quantize_q8_1(to_dev(x), to_dev(w), eps, M, K, xq)
    torch.cuda.synchronize()
    return xq.cpu().numpy()


def check(x, w, eps, where):
    got = run(x, w, eps)
    exp = oracle.rmsnorm_quantize_q8_1(x, w, eps).reshape(-1)
    if not np.array_equal(got, exp):
        M, K = x.shape
        blk = np.argwhere(got.reshape(M, -1, 36) != exp.reshape(M, -1, 36))[0]
        raise AssertionError(f"{where}: bytes differ, first at row {blk[0]} block {blk[1]} byte {blk[2]}")


# hidden sizes of the pages' models (1536, 4096, 5120) plus ragged and large K
@pytest.mark.parametrize("K", [32, 256, 1536, 4096, 5120, 12288, 17408, 32768])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_bytes_match_oracle(K, M):
    rng = np.random.default_rng(K * 10 + M)
    x = (rng.standard_normal((M, K)) * rng.uniform(0.1, 30.0, (M, 1))).astype(np.float32)
    w = rng.uniform(0.2, 2.0, K).astype(np.float32)
    check(x, w, 1e-6, f"K={K} M={M}")


@pytest.mark.parametrize("eps", [0.0, 1e-5, 1.0])
def test_eps_and_edge_rows(eps):
    K = 2048
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, K)).astype(np.float32)
    x[1] = 0.0                      # zero row: all-zero blocks (eps > 0) or 0/0 -> NaN codes skipped
    x[2, :] = 1.0
    x[2, 0] = 2.0 ** 12             # a sum whose fp32 value depends on the order
    x[2, 1:8] = 0.0                 # group 0 = 2^24, then groups of 8: serial 2^24 + ...
    x[3] *= 1e-20                   # tiny values
    x[4, 100:132] = 0.0             # one all-zero block inside a row
    x[5] = np.float32(3.0)          # constant row
    w = np.ones(K, np.float32)
    if eps == 0.0:
        x[1] = 1.0                  # keep 0/0 out of the contract
    check(x, w, eps, f"edge rows eps={eps}")


def test_equals_quantizer_of_oracle_norm():
    """The fused kernel's bytes are the standalone GPU quantizer's bytes on the
    oracle's normalized rows: the fusion changes no decision."""
    import torch
    M, K = 4, 4096
    rng = np.random.default_rng(3)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, K).astype(np.float32)
    xn, _ = oracle.rmsnorm(x, w, 1e-6)
    xq = torch.empty(qd.qdot_q8_1_bytes(M, K), dtype=torch.uint8, device=dev())
    qd.qdot_quantize_q8_1(to_dev(xn), M, K, xq)
    torch.cuda.synchronize()
    assert np.array_equal(run(x, w, 1e-6), xq.cpu().numpy())


def test_serial_group_order_row():
    """The row worked out by hand in the oracle's pins (Kestrel #18 section
    3.6 order: ss = 2^24 + 8, where the pairwise block tree gives 2^24 + 14),
    repeated along a long row and mixed with ordinary rows, so that the
    kernel's serial pass over the group sums is what decides the bytes."""
    K = 4096
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, K)).astype(np.float32)
    x[1] = 0.0
    x[1, 0:8] = [2.0 ** 12, 1, 1, 1, 1, 1, 1, 1]
    x[1, 8::8] = 1.0
    w = rng.uniform(0.5, 1.5, K).astype(np.float32)
    _, ss = oracle.rmsnorm(x, w, 0.0)
    assert ss[1] == np.float32(2.0 ** 24 + 8)   # every further + 1 is a tie that rounds back
    check(x, w, 0.0, "serial order row")
