"""GPU parity of qdot_attn_decode_kv4 (decode attention over the 4-bit KV
cache) against the CPU oracle, through the C ABI.

Bar: |out - oracle| <= 1e-4 * max |v| of the head's value rows, on every
output.  The scores take one fp32 rounding of the oracle's exact fp64 value;
expf, the fp32 sums over a 256-token chunk and the chunk combine add a few
1e-6 relative to the largest value each; the bound leaves a factor of about
three over that estimate.  T = 1 is exact.  Outputs are NaN-poisoned before
each call and must be fully written; two calls give the same bits.
"""
import math

import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import binding as qd
from quant_integer_dot_amd import synth

from gpu_util import dev, quantize, to_dev

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qd.load()


def run(qd_q, Hq, Kd, Vd, Hkv, T, scale, ws=None):
    import torch
    out = torch.full((Hq, D), float("nan"), dtype=torch.float32, device=dev())
    nb = qd.qdot_attn_kv4_workspace_bytes(Hq, T)
    if ws is None:
        ws = torch.full((nb // 4,), float("nan"), dtype=torch.float32, device=dev())
    qd.qdot_attn_decode_kv4(qd_q, Hq, Kd, Vd, Hkv, T, D, scale, out, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def vmax(V, Hq, Hkv):
    """max |v| of the value rows each query head reads."""
    G = Hq // Hkv
    rows = V.reshape(Hkv, -1, D // 32, 18)
    d = np.abs(rows[..., 0:2].copy().view(np.float16).astype(np.float64))[..., 0]
    per_kv = (d * 8).reshape(Hkv, -1).max(axis=1)
    return np.repeat(per_kv, G)


def check(out, o64, V, Hq, Hkv, where):
    assert not np.isnan(out).any(), f"{where}: output not fully written"
    tol = 1e-4 * vmax(V, Hq, Hkv)[:, None]
    err = np.abs(out.astype(np.float64) - o64)
    bad = err > tol
    if bad.any():
        h, d = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {bad.sum()} outputs off; first ({h},{d}): gpu={out[h, d]!r} "
                             f"oracle={o64[h, d]!r} tol={tol[h, 0]:.3g}")


def case(Hq, Hkv, T, seed, qscale=1.0):
    K = synth.kv4_cache(Hkv, T, D, (seed, 1))
    V = synth.kv4_cache(Hkv, T, D, (seed, 2))
    x = synth.activations(Hq, D, (seed, 3)) * np.float32(qscale)
    xqd, xq = quantize(x)
    return K, V, xqd, xq


@pytest.mark.parametrize("Hq,Hkv,T", [(4, 1, 1), (4, 1, 255), (8, 2, 256), (8, 2, 257), (6, 2, 513),
                                      (32, 8, 1000), (8, 1, 700), (5, 5, 300), (14, 2, 777), (3, 1, 2049)])
def test_parity(Hq, Hkv, T):
    """Several 256-token chunks and a ragged tail, every group size 1..8 in
    the Qwen3 / Llama shapes and odd ones."""
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 100 + T + Hq)
    out = run(xqd, Hq, to_dev(K), to_dev(V), Hkv, T, scale)
    o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, Hq, Hkv, f"Hq={Hq} Hkv={Hkv} T={T}")
    if T == 1:
        assert np.array_equal(out.astype(np.float64), o64), "T = 1 returns the value row exactly"


def test_peaked_scores():
    """A query scaled up 40x: scores spread over about +-100, the softmax
    concentrates on a few tokens in different chunks."""
    Hq, Hkv, T = 8, 2, 1500
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 7, qscale=40.0)
    out = run(xqd, Hq, to_dev(K), to_dev(V), Hkv, T, scale)
    o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    assert sc.max() - sc.min() > 50
    check(out, o64, V, Hq, Hkv, "peaked")


@pytest.mark.parametrize("Hq,Hkv,T", [(32, 8, 28672), (32, 8, 32768), (12, 2, 32768)])
def test_full_size(Hq, Hkv, T):
    """Qwen3-8B heads (32 query, 8 KV, D = 128) at the long-context lengths
    of the pages (28K and 32K tokens) and Qwen2.5-1.5B heads (12 query, 2 KV)
    at 32K, every output against the oracle; bitwise deterministic."""
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 11)
    Kd, Vd = to_dev(K), to_dev(V)
    out = run(xqd, Hq, Kd, Vd, Hkv, T, scale)
    o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, Hq, Hkv, f"T={T}")
    again = run(xqd, Hq, Kd, Vd, Hkv, T, scale)
    assert np.array_equal(out.view(np.uint32), again.view(np.uint32))


def test_workspace_reused_for_a_shorter_context():
    """One workspace, a long call then a shorter one: each result is its own."""
    import torch
    Hq, Hkv = 8, 2
    scale = np.float32(0.1)
    ws = torch.full((qd.qdot_attn_kv4_workspace_bytes(Hq, 1300) // 4,), float("nan"), dtype=torch.float32,
                    device=dev())
    for T in (1300, 400):
        K, V, xqd, xq = case(Hq, Hkv, T, 300 + T)
        out = run(xqd, Hq, to_dev(K), to_dev(V), Hkv, T, scale, ws=ws)
        o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
        check(out, o64, V, Hq, Hkv, f"reuse T={T}")


def test_offset_cache_views():
    """K and V at 8-byte (not 256-byte) offsets inside larger buffers."""
    import torch
    Hq, Hkv, T = 4, 1, 300
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 55)
    Kb = torch.zeros(K.size + 64, dtype=torch.uint8, device=dev())
    Vb = torch.zeros(V.size + 64, dtype=torch.uint8, device=dev())
    Kb[8:8 + K.size] = to_dev(K.reshape(-1))
    Vb[24:24 + V.size] = to_dev(V.reshape(-1))
    out = run(xqd, Hq, Kb.data_ptr() + 8, Vb.data_ptr() + 24, Hkv, T, scale)
    o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, Hq, Hkv, "offset views")


def test_million_token_context():
    """T = 1,000,003 (3907 chunks, a ragged tail): the combine joins 3907
    partials per head (245 per residue); every output against the oracle."""
    Hq, Hkv, T = 4, 1, 1_000_003
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 21)
    out = run(xqd, Hq, to_dev(K), to_dev(V), Hkv, T, scale)
    o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, Hq, Hkv, "T=1000003")


def test_negative_and_large_scale():
    """A negative scale (softmax of -s) and a large one (weights nearly
    one-hot) are ordinary finite arguments."""
    Hq, Hkv, T = 8, 2, 600
    K, V, xqd, xq = case(Hq, Hkv, T, 23)
    Kd, Vd = to_dev(K), to_dev(V)
    for scale in (np.float32(-0.05), np.float32(2.0)):
        out = run(xqd, Hq, Kd, Vd, Hkv, T, scale)
        o64, _ = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
        check(out, o64, V, Hq, Hkv, f"scale={scale}")
