"""GPU parity of qdot_attn_decode_kv4 (decode attention over the 4-bit KV
cache) against the CPU oracle, through the C ABI.

Bar, per output element d of head h, with u = 2^-24 and the oracle's fp64
scores s_t and weights p_t = e^(s_t - max s):

  A_d   = sum_t p_t |v_t[d]| / sum_t p_t   (the scale of the output's terms)
  |out - oracle| <= A_d * u * (2 (6 smax + 6) + n_num + n_den + 2)

a first-order worst-case bound on the kernel's fp32 arithmetic: each weight
carries the roundings of s_t and of the maxima, two subtractions and two
expf calls (2 ulp each), at most (6 smax + 6) u relative with smax the
largest |s_t| of the head, and a relative change e of every weight moves a
convex combination by at most 2 e A_d; the numerator is summed in chains of
n_num = 32 (tokens of a half-wave) + 1 (the two half-waves) + 3 (waves) +
ceil(chunks / 16) (partials of a residue) + 15 (residues) additions and the
denominator in n_den = 6 + 3 +
ceil(chunks / 512) + 6 + 7, each addition adding at most u of the sum of the
absolute terms; one more rounding for the division.  On top, the RMS over a
call's outputs of |out - oracle| / A_d must stay under u (4 + sqrt(n_num +
n_den)): rounding errors of long sums grow like the square root of the chain
length in practice (the probabilistic model of rounding error growth), so a
systematic error of a few 1e-7 relative, which the worst-case bound would
admit, fails here.  T = 1 is exact.  Outputs are NaN-poisoned before each
call and must be fully written; two calls give the same bits.
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


U = 2.0 ** -24


def term_scale(V, scores, Hq, Hkv):
    """A[h][d] = sum_t p_t |v_t[d]| / sum_t p_t (fp64, from the oracle's
    scores), and the largest |s_t| of each head."""
    G = Hq // Hkv
    T = scores.shape[1]
    A = np.zeros((Hq, D))
    smax = np.abs(scores).max(axis=1)
    rows = V.reshape(Hkv, T, D // 32, 18)
    for kvh in range(Hkv):
        p = np.exp(scores[kvh * G:(kvh + 1) * G] - scores[kvh * G:(kvh + 1) * G].max(axis=1, keepdims=True))
        acc = np.zeros((G, D))
        for t0 in range(0, T, 65536):
            blk = rows[kvh, t0:t0 + 65536]
            dv = blk[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
            codes = blk[..., 2:]
            lo = (codes & 15).astype(np.float32) - 8
            hi = (codes >> 4).astype(np.float32) - 8
            v = np.concatenate([lo, hi], axis=2) * dv[..., None]      # [t][block][32]
            acc += p[:, t0:t0 + 65536] @ np.abs(v.reshape(-1, D)).astype(np.float64)
        A[kvh * G:(kvh + 1) * G] = acc / p.sum(axis=1, keepdims=True)
    return A, smax


def check(out, o64, V, scores, Hq, Hkv, where):
    assert not np.isnan(out).any(), f"{where}: output not fully written"
    T = scores.shape[1]
    chunks = -(-T // 256)
    n_num = 32 + 1 + 3 + -(-chunks // 16) + 15
    n_den = 6 + 3 + -(-chunks // 512) + 6 + 7
    A, smax = term_scale(V, scores, Hq, Hkv)
    tol = A * U * (2 * (6 * smax[:, None] + 6) + n_num + n_den + 2)
    err = np.abs(out.astype(np.float64) - o64)
    bad = err > tol
    if bad.any():
        h, d = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {bad.sum()} outputs off; first ({h},{d}): gpu={out[h, d]!r} "
                             f"oracle={o64[h, d]!r} tol={tol[h, d]:.3g}")
    live = A > 0
    rms = np.sqrt(np.mean((err[live] / A[live]) ** 2))
    assert rms <= U * (4 + np.sqrt(n_num + n_den)), f"{where}: RMS relative error {rms:.3g}"


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
    o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, sc, Hq, Hkv, f"Hq={Hq} Hkv={Hkv} T={T}")
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
    check(out, o64, V, sc, Hq, Hkv, "peaked")


@pytest.mark.parametrize("Hq,Hkv,T", [(32, 8, 28672), (32, 8, 32768), (12, 2, 32768)])
def test_full_size(Hq, Hkv, T):
    """Qwen3-8B heads (32 query, 8 KV, D = 128) at the long-context lengths
    of the pages (28K and 32K tokens) and Qwen2.5-1.5B heads (12 query, 2 KV)
    at 32K, every output against the oracle; bitwise deterministic."""
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 11)
    Kd, Vd = to_dev(K), to_dev(V)
    out = run(xqd, Hq, Kd, Vd, Hkv, T, scale)
    o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, sc, Hq, Hkv, f"T={T}")
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
        o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
        check(out, o64, V, sc, Hq, Hkv, f"reuse T={T}")


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
    o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, sc, Hq, Hkv, "offset views")


def test_million_token_context():
    """T = 1,000,003 (3907 chunks, a ragged tail): the combine joins 3907
    partials per head (245 per residue); every output against the oracle."""
    Hq, Hkv, T = 4, 1, 1_000_003
    scale = np.float32(1 / math.sqrt(D))
    K, V, xqd, xq = case(Hq, Hkv, T, 21)
    out = run(xqd, Hq, to_dev(K), to_dev(V), Hkv, T, scale)
    o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
    check(out, o64, V, sc, Hq, Hkv, "T=1000003")


def test_negative_and_large_scale():
    """A negative scale (softmax of -s) and a large one (weights nearly
    one-hot) are ordinary finite arguments."""
    Hq, Hkv, T = 8, 2, 600
    K, V, xqd, xq = case(Hq, Hkv, T, 23)
    Kd, Vd = to_dev(K), to_dev(V)
    for scale in (np.float32(-0.05), np.float32(2.0)):
        out = run(xqd, Hq, Kd, Vd, Hkv, T, scale)
        o64, sc = oracle.attn_decode_kv4(xq, Hq, K, V, Hkv, T, D, float(scale))
        check(out, o64, V, sc, Hq, Hkv, f"scale={scale}")
