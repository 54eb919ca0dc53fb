"""GPU: the grouped call (qdot_qmatmul_multi) against single-matrix calls and
the oracle.  Each matrix of a group must come out bitwise equal to its own
qdot_qmatmul call (same tile code, K split and summation order), so the
single-call parity tests carry over; sampled rows are also checked against
the oracle directly."""
import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd
from quant_integer_dot_amd import synth

from gpu_util import assert_close, dev, qmatmul, quantize, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


def run_multi(Wds, types, Ns, K, xqd, M):
    import torch
    ys = [torch.full((M, N), float("nan"), dtype=torch.float32, device=dev()) for N in Ns]
    qd.qdot_qmatmul_multi(Wds, types, Ns, K, xqd, M, ys)
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in ys]


def check_group(mats, K, M, seed, n_oracle_rows=6, signed_scales=False):
    """n_oracle_rows: sampled rows of each matrix checked against the oracle
    (None: every row)."""
    Ws = [synth.weights(t, N, K, (2026, 80, seed, i), signed_scales=signed_scales)
          for i, (N, t) in enumerate(mats)]
    Wds = [to_dev(W) for W in Ws]
    x = synth.activations(M, K, (2026, 80, seed, K, M))
    xqd, xq = quantize(x)
    types = [t for _, t in mats]
    Ns = [N for N, _ in mats]
    ys = run_multi(Wds, types, Ns, K, xqd, M)
    for i, (N, t) in enumerate(mats):
        y1, _ = qmatmul(Wds[i], t, N, K, xqd, M)
        assert np.array_equal(ys[i].view(np.uint32), y1.view(np.uint32)), \
            f"matrix {i} ({synth.TYPE_NAMES[t]} {N}x{K}) M={M}: group != single call"
        if n_oracle_rows is None:
            y64, _, _ = oracle.qmatmul(Ws[i], t, N, K, xq, M)
            assert_close(ys[i], y64, f"group matrix {i} M={M}")
            continue
        rows = np.unique(np.concatenate([np.random.default_rng(seed + i).integers(0, N, n_oracle_rows),
                                         [0, N - 1]]))
        y64, _ = oracle.qmatmul_rows(Ws[i], t, N, K, xq, M, rows)
        assert_close(ys[i][:, rows], y64, f"group matrix {i} M={M}")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_qkv_mixed_q4k_q6k(M):
    """Q (Q4_K), K (Q4_K), V (Q6_K), ragged row counts, one launch."""
    check_group([(200, synth.Q4_K), (70, synth.Q4_K), (33, synth.Q6_K)], 1024, M, seed=M)


@pytest.mark.parametrize("M", [1, 5, 8])
def test_group_q4k_q6k_long_rows(M):
    """Q4_K and Q6_K matrices with 48-superblock rows (K = 12288) in one
    group (the Q4_K ones on MFMA tiles, the group being small): each output bitwise equal
    to its own single call."""
    check_group([(96, synth.Q4_K), (40, synth.Q6_K), (33, synth.Q4_K)], 12288, M, seed=100 + M)


QKV_8B = [(4096, synth.Q4_K), (1024, synth.Q4_K), (1024, synth.Q6_K)]
GATE_UP_8B = [(12288, synth.Q4_K), (12288, synth.Q4_K)]


def headline_tiles(mats, K, M):
    return [qd.qdot_multi_kernel_name([t for _, t in mats], [N for N, _ in mats], K, M, i)
            for i in range(len(mats))]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gate_up_full_size(M):
    """Gate and up of the 8B FFN (two 12288 x 4096 Q4_K) in one launch, as
    the benchmark step runs them at every M: the dot4 tile at M = 1, 2 and
    the MFMA tile from M = 3 (asserted through the tile names), every output
    against the oracle."""
    tiles = headline_tiles(GATE_UP_8B, 4096, M)
    kind = "qmv_dot4" if M <= 2 else "qmv_mfma"
    assert tiles == [f"{kind}<Q4_K,{M}>"] * 2, tiles
    check_group(GATE_UP_8B, 4096, M, seed=10 + M, n_oracle_rows=None)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_qkv_full_size(M):
    """q, k (Q4_K, MFMA tiles at every M) and v (Q6_K, dot4 tile; its 16-row
    MFMA tile at M = 7, 8) of the 8B attention in one launch, as the
    benchmark step runs them; every output against the oracle."""
    tiles = headline_tiles(QKV_8B, 4096, M)
    v_tile = f"qmv_mfma<Q6_K,{M}>" if M >= 7 else f"qmv_dot4<Q6_K,{M}>"
    assert tiles == [f"qmv_mfma<Q4_K,{M}>"] * 2 + [v_tile], tiles
    check_group(QKV_8B, 4096, M, seed=20 + M, n_oracle_rows=None)


@pytest.mark.parametrize("M", [1, 3, 8])
def test_headline_groups_signed_scales(M):
    """The same two groups with weights whose fp16 d and dmin carry random
    signs (the workloads draw them positive)."""
    check_group(QKV_8B, 4096, M, seed=90 + M, n_oracle_rows=None, signed_scales=True)
    check_group(GATE_UP_8B, 4096, M, seed=95 + M, n_oracle_rows=64, signed_scales=True)


TP8_FFN = [(1536, synth.Q4_K), (1536, synth.Q4_K)]  # one GPU's gate and up under 8-way TP


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_tp8_shard_shapes_every_row(M):
    """One GPU's share of the 8B FFN under 8-way tensor parallelism, as the
    benchmark's shard rows run it: gate+up (2 x 1536 x 4096 Q4_K) grouped and
    down (4096 x 1536 Q6_K, six superblocks a row) alone; every output
    against the oracle."""
    check_group(TP8_FFN, 4096, M, seed=200 + M, n_oracle_rows=None)
    W = synth.weights(synth.Q6_K, 4096, 1536, (2026, 81, M))
    x = synth.activations(M, 1536, (2026, 81, 1536, M))
    xqd, xq = quantize(x)
    y, _ = qmatmul(to_dev(W), synth.Q6_K, 4096, 1536, xqd, M)
    y64, _, _ = oracle.qmatmul(W, synth.Q6_K, 4096, 1536, xq, M)
    assert_close(y, y64, f"down shard 4096x1536 M={M}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_q4_0_with_q8_0(M):
    check_group([(130, synth.Q4_0), (64, synth.Q8_0), (17, synth.Q4_0)], 768, M, seed=30 + M)


@pytest.mark.parametrize("M", [2, 7])
def test_unfused_mix_runs_per_type(M):
    """IQ4_XS with Q4_K and Q8_0: one launch per type, same results."""
    check_group([(48, synth.IQ4_XS), (40, synth.Q4_K), (24, synth.Q8_0), (16, synth.IQ4_XS)], 512, M,
                seed=40 + M)


@pytest.mark.parametrize("M", [9, 16, 17, 40, 100])
def test_above_decode_launches_each(M):
    """Above M = 8 each matrix is its own launch: Q4_K and IQ4_XS on the
    16-row decode tile up to M = 16, Q6_K on the mid-batch kernel."""
    check_group([(96, synth.Q4_K), (50, synth.Q6_K), (80, synth.IQ4_XS)], 512, M, seed=50 + M)


def test_single_matrix_group():
    check_group([(300, synth.IQ4_XS)], 5120, 3, seed=60)
