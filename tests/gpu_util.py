"""Helpers for the GPU parity tests: device buffers and calls through the C ABI."""
import numpy as np

import oracle
from quant_integer_dot_amd import binding as qd


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def quantize(x_h):
    """GPU quantizer on host fp32 [M][K]; returns (device tensor, host bytes)."""
    import torch
    M, K = x_h.shape
    xd = to_dev(x_h.astype(np.float32))
    xq = torch.full((qd.qdot_q8_1_bytes(M, K),), 0xA5, dtype=torch.uint8, device=dev())
    qd.qdot_quantize_q8_1(xd, M, K, xq)
    torch.cuda.synchronize()
    return xq, xq.cpu().numpy()


def qmatmul(Wd, wtype, N, K, xqd, M, dump=False):
    """Runs the GPU matmul with a NaN-poisoned y; returns (y host, isums host|None)."""
    import torch
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev())
    if dump:
        isums = torch.full((qd.qdot_isum_count(wtype, N, K, M),), -0x5A5A5A5A, dtype=torch.int32,
                           device=dev())
        qd.qdot_qmatmul_dump_isums(Wd, wtype, N, K, xqd, M, y, isums)
        torch.cuda.synchronize()
        sub = 16 if wtype == qd.QDOT_Q6_K else 32
        return y.cpu().numpy(), isums.cpu().numpy().reshape(M, N, K // sub)
    qd.qdot_qmatmul(Wd, wtype, N, K, xqd, M, y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), None


def assert_close(y_gpu, y64, where=""):
    """Every output within relative 1e-5 of the oracle's fp64 value (exact
    zeros must be exact).  The GPU keeps every scale product exact and sums
    in fp64, so the only sizable error is the final fp32 rounding (2^-24)."""
    assert not np.isnan(y_gpu).any(), f"{where}: output not fully written"
    err = np.abs(y_gpu.astype(np.float64) - y64)
    bad = err > 1e-5 * np.abs(y64)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {bad.sum()} outputs off; first {tuple(i)}: "
                             f"gpu={y_gpu[tuple(i)]!r} oracle={y64[tuple(i)]!r}")
