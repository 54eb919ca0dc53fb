"""CPU pins of the int4-KV decode-attention oracle (oracle_attn_decode_kv4):
closed forms, the layout read bit by bit, the grouped-head mapping, and its
scores against the independently pinned Q4_0 matmul oracle."""
import math

import numpy as np
import pytest

import oracle
from quant_integer_dot_amd import synth

Q4_0 = oracle.Q4_0


def pack_rows(codes, d):
    """Q4_0 rows from element codes [R][D] (0..15) and block scales [R][D/32],
    packed by hand from the layout: byte i of a block holds element i in its
    low nibble and element 16 + i in its high nibble, after the fp16 scale."""
    codes = np.asarray(codes, dtype=np.int64)
    R, D = codes.shape
    out = np.zeros((R, D // 32, 18), dtype=np.uint8)
    out[:, :, 0:2] = np.asarray(d, dtype=np.float16).reshape(R, D // 32, 1).view(np.uint8)
    c = codes.reshape(R, D // 32, 32)
    out[:, :, 2:] = (c[:, :, :16] | (c[:, :, 16:] << 4)).astype(np.uint8)
    return out.reshape(R, D // 32 * 18)


def dequant_rows(rows, D):
    """Values of Q4_0 rows through the pinned Q4_0 weight oracle: two rows of
    128 (or one of 256) make one 256-element Q4_0 group."""
    R = rows.shape[0]
    flat = rows.reshape(-1)
    n = flat.size // 144
    return oracle.dequant(flat, Q4_0, n, 256).reshape(R, D)


def test_single_token_returns_its_value_row():
    """T = 1: the only weight is 1, so out = V row of the head's KV head."""
    Hq, Hkv, D = 4, 2, 128
    K = synth.kv4_cache(Hkv, 1, D, (1, 1))
    V = synth.kv4_cache(Hkv, 2, D, (1, 2))[:, :1].copy()
    q = oracle.quantize_q8_1(synth.activations(Hq, D, (1, 3)))
    out, _ = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, 1, D, 1 / math.sqrt(D))
    vv = dequant_rows(np.concatenate([V[0], V[1]]), D)
    for h in range(Hq):
        assert np.array_equal(out[h], vv[h // 2])


def test_equal_keys_average_the_values():
    """All K rows equal: every weight is 1/T, out = mean of the V rows."""
    Hq, Hkv, T, D = 2, 1, 10, 128
    K = np.repeat(synth.kv4_cache(1, 1, D, (2, 1)), T, axis=1)
    V = synth.kv4_cache(1, T, D, (2, 2))
    q = oracle.quantize_q8_1(synth.activations(Hq, D, (2, 3)))
    out, sc = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, T, D, 0.3)
    assert np.all(sc == sc[:, :1])
    mean = dequant_rows(V[0], D).mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(out[h], mean, rtol=0, atol=1e-15)


def test_two_tokens_sigmoid_closed_form():
    """Query of ones (codes 127, D = fp16(1/127)); key 0 has every element
    d = 1, code 9 (value 1), key 1 code 8 (value 0): s0 = scale * 4 * D * 32 *
    127, s1 = 0; values 0.5 and 0, so out = 0.5 * sigmoid(s0)."""
    D = 128
    q = oracle.quantize_q8_1(np.ones((1, D), dtype=np.float32))
    Dq = float(np.float16(1 / 127))
    K = pack_rows([[9] * D, [8] * D], np.ones((2, 4))).reshape(1, 2, 72)
    V = pack_rows([[9] * D, [8] * D], np.full((2, 4), 0.5)).reshape(1, 2, 72)
    scale = 1 / math.sqrt(D)
    out, sc = oracle.attn_decode_kv4(q, 1, K, V, 1, 2, D, scale)
    s0 = scale * 4 * Dq * 32 * 127
    assert sc[0, 0] == s0 and sc[0, 1] == 0.0
    np.testing.assert_allclose(out[0], 0.5 / (1 + math.exp(-s0)), rtol=1e-15)


@pytest.mark.parametrize("i0", [0, 3, 15, 16, 19, 31, 37, 127])
def test_key_element_positions(i0):
    """One-hot query at element i0 and one key whose only nonzero value sits
    at i0: the score is scale * dK * fp16(1/127) * 127 * c; a key with the
    value one element over scores 0 (the nibble and byte order of the layout)."""
    D, c = 128, 5
    x = np.zeros((1, D), dtype=np.float32)
    x[0, i0] = 1.0
    q = oracle.quantize_q8_1(x)
    codes = np.full((2, D), 8)
    codes[0, i0] = 8 + c
    codes[1, (i0 + 1) % D] = 8 + c
    K = pack_rows(codes, np.full((2, 4), 0.25)).reshape(1, 2, 72)
    V = synth.kv4_cache(1, 2, D, (3, i0))
    _, sc = oracle.attn_decode_kv4(q, 1, K, V, 1, 2, D, 0.5)
    assert sc[0, 0] == 0.5 * 0.25 * float(np.float16(1 / 127)) * 127 * c
    assert sc[0, 1] == 0.0


def test_value_element_positions():
    """T = 1 with hand-packed value codes: out[d] = dV_b * (code_d - 8)."""
    D = 128
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, (1, D))
    dv = np.array([[0.5, 0.25, 2.0, 0.125]])
    V = pack_rows(codes, dv).reshape(1, 1, 72)
    K = synth.kv4_cache(1, 1, D, (4, 1))
    q = oracle.quantize_q8_1(synth.activations(1, D, (4, 2)))
    out, _ = oracle.attn_decode_kv4(q, 1, K, V, 1, 1, D, 0.1)
    want = np.repeat(dv, 32, axis=1)[0] * (codes[0] - 8)
    assert np.array_equal(out[0], want)


def test_grouped_heads_read_their_kv_head():
    """Hq = 6 over Hkv = 2: heads 0-2 read KV head 0 (all values +1), heads
    3-5 KV head 1 (all -1), whatever the keys."""
    Hq, Hkv, T, D = 6, 2, 9, 128
    K = synth.kv4_cache(Hkv, T, D, (5, 1))
    V = np.concatenate([pack_rows(np.full((T, D), 9), np.ones((T, 4))).reshape(1, T, 72),
                        pack_rows(np.full((T, D), 7), np.ones((T, 4))).reshape(1, T, 72)])
    q = oracle.quantize_q8_1(synth.activations(Hq, D, (5, 2)))
    out, _ = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, T, D, 1 / math.sqrt(D))
    np.testing.assert_allclose(out[:3], 1.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[3:], -1.0, rtol=0, atol=1e-15)


def test_token_order_does_not_matter():
    """Permuting the tokens (K and V rows together) leaves the output
    unchanged up to fp64 rounding; permuting V alone changes it."""
    Hq, Hkv, T, D = 4, 1, 33, 128
    K = synth.kv4_cache(Hkv, T, D, (6, 1))
    V = synth.kv4_cache(Hkv, T, D, (6, 2))
    q = oracle.quantize_q8_1(synth.activations(Hq, D, (6, 3)) * 3)
    perm = np.random.default_rng(8).permutation(T)
    a, _ = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, T, D, 1 / math.sqrt(D))
    b, _ = oracle.attn_decode_kv4(q, Hq, K[:, perm].copy(), V[:, perm].copy(), Hkv, T, D, 1 / math.sqrt(D))
    c, _ = oracle.attn_decode_kv4(q, Hq, K, V[:, perm].copy(), Hkv, T, D, 1 / math.sqrt(D))
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    assert np.abs(a - c).max() > 1e-3


def test_scores_match_the_q4_0_matmul_oracle():
    """D = 256: a key row is one 256-element Q4_0 group, so the scores are
    scale times the pinned Q4_0 matmul of the keys with the query rows
    (the same exact terms in the same order: bit for bit)."""
    Hq, Hkv, T, D = 4, 2, 37, 256
    K = synth.kv4_cache(Hkv, T, D, (9, 1))
    V = synth.kv4_cache(Hkv, T, D, (9, 2))
    x = synth.activations(Hq, D, (9, 3))
    q = oracle.quantize_q8_1(x)
    scale = 0.0625
    _, sc = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, T, D, scale)
    for g in range(Hkv):
        y64, _, _ = oracle.qmatmul(K[g].copy(), Q4_0, T, D, q[2 * g:2 * g + 2].copy(), 2)
        assert np.array_equal(sc[2 * g:2 * g + 2], scale * y64)


def test_softmax_weights_are_a_distribution():
    """Against softmax computed from the returned scores by the library
    routine (scipy): the output is that weighting of the dequantized values."""
    from scipy.special import softmax
    Hq, Hkv, T, D = 4, 2, 50, 128
    K = synth.kv4_cache(Hkv, T, D, (10, 1))
    V = synth.kv4_cache(Hkv, T, D, (10, 2))
    q = oracle.quantize_q8_1(synth.activations(Hq, D, (10, 3)) * 4)
    out, sc = oracle.attn_decode_kv4(q, Hq, K, V, Hkv, T, D, 1 / math.sqrt(D))
    for h in range(Hq):
        p = softmax(sc[h])
        vv = dequant_rows(V[h // 2], D)
        np.testing.assert_allclose(out[h], p @ vv, rtol=0, atol=1e-13)


def test_bad_arguments():
    """Heads that do not group evenly, and a row length off the block size,
    are rejected."""
    q = np.zeros(3 * 4 * 36, dtype=np.uint8)
    kv = np.zeros(2 * 72, dtype=np.uint8)
    with pytest.raises(ValueError):
        oracle.attn_decode_kv4(q, 3, kv, kv, 2, 1, 128, 1.0)
    L = oracle.lib()
    out = np.zeros(64, dtype=np.float64)
    assert L.oracle_attn_decode_kv4(oracle._ptr(q), 1, oracle._ptr(kv), oracle._ptr(kv), 1, 1, 48, 1.0,
                                    oracle._ptr(out), None) == -1
    assert L.oracle_attn_decode_kv4(oracle._ptr(q), 1, oracle._ptr(kv), oracle._ptr(kv), 1, 0, 128, 1.0,
                                    oracle._ptr(out), None) == -1
