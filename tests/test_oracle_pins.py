"""Pins of the CPU oracle against things other than itself.

- binary16 decode: exhaustive against numpy's float16 (a library routine).
- binary16 encode: against numpy's float32->float16 rounding on many values.
- Q8_1 quantizer: invariants of the stated reading (amax maps to +-127, round
  to nearest with ties away from zero, |x - d*q| <= d/2, S = fp16(D*sum q)).
- weight decoders: test-side *encoders* (the inverse mapping, written from the
  layout readings) feed chosen field values; the oracle must return exactly
  the values the fields define.
- matmul and sub-block sums: exact Fractions evaluated from field values
  (brute force on tiny inputs), the dequantize-then-dot textbook identity, a
  one-hot closed form and the special cases.
- the pages' statistical anchor: about 0.5 % RMS against fp32 SGEMV with the
  argmax kept (golden fixture with its citation).
- RMSNorm (the fused producer of the Q8_1 activations): a closed form on
  constant rows, exact power-of-two scale invariances, the fp64 formula within
  the fp32 error bound, and the page's summation order (8-element group sums
  added left to right) on a row worked out by hand where other orders give
  other fp32 sums.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import qfields as qf

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TYPES = [qf.Q4_K, qf.Q6_K, qf.IQ4_XS, qf.Q4_0, qf.Q8_0]


# ------------------------------------------------------------- binary16
def test_half_decode_exhaustive(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_half_encode_matches_numpy(oracle_lib):
    rng = np.random.default_rng(11)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9,
            2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 0.1, 1 / 3]
    # exact ties of the binary16 grid at many exponents
    for e in range(-24, 16):
        for m in (1024, 1025, 2047):
            vals.append((m + 0.5) * 2.0 ** (e - 10))
    vals += list((rng.standard_normal(20000) * np.exp(rng.uniform(-20, 12, 20000))))
    x32 = np.array(vals, dtype=np.float32)
    ref = x32.astype(np.float16).view(np.uint16)
    got = np.array([oracle_lib.double_to_half(float(v)) for v in x32], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x32[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------- Q8_1 quantizer
def _q8_fields(xq, M, K):
    blk = xq.reshape(M, K // 32, 36)
    D = blk[:, :, 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    S = blk[:, :, 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
    q = blk[:, :, 4:].view(np.int8).astype(np.int64)
    return D, S, q


def test_q8_1_invariants(oracle_lib):
    rng = np.random.default_rng(5)
    M, K = 3, 2048
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[1, 64:96] = 0.0                                    # amax == 0 block
    x[2, 96:128] *= np.float32(1e-4)                     # subnormal fp16 d
    xq = oracle_lib.quantize_q8_1(x)
    D, S, q = _q8_fields(xq, M, K)
    xb = x.reshape(M, K // 32, 32).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    for m in range(M):
        for b in range(K // 32):
            if amax[m, b] == 0:
                assert D[m, b] == 0 and S[m, b] == 0 and not q[m, b].any()
                continue
            d32 = float(np.float32(amax[m, b]) / np.float32(127.0))
            # D is the nearest binary16 to d32 (numpy's rounding as the reference)
            assert D[m, b] == float(np.float16(np.float32(d32)))
            i = int(np.argmax(np.abs(xb[m, b])))
            assert q[m, b, i] == (127 if xb[m, b, i] > 0 else -127)
            # round-to-nearest bound: |x/d32 - q| <= 1/2 (+ fp32 division ulp)
            err = np.abs(xb[m, b] / d32 - q[m, b])
            assert err.max() <= 0.5 + 1e-5
            assert np.all(np.abs(q[m, b]) <= 127)
            assert np.all(np.sign(q[m, b]) * np.sign(xb[m, b]) >= 0)
            assert S[m, b] == float(np.float16(D[m, b] * q[m, b].sum()))


def test_q8_1_ties_round_away_from_zero(oracle_lib):
    # amax = 127 makes d32 == 1.0 exactly, so x/d32 == x and ties are exact.
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [0.5, -0.5, 1.5, -1.5, 2.5, -2.5, 126.5, -126.5]
    x[0, 9:12] = [0.49999997, 2.4999998, -3.5000002]
    D, S, q = _q8_fields(oracle_lib.quantize_q8_1(x), 1, 32)
    assert D[0, 0] == 1.0
    assert list(q[0, 0, :12]) == [127, 1, -1, 2, -2, 3, -3, 127, -127, 0, 2, -4]


def _rne32(v):
    """Exact round-to-nearest-even of a Fraction to binary32 (normal range)."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sgn, a = (-1 if v < 0 else 1), abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while a / Fraction(2) ** e >= 2:
        e += 1
    while a / Fraction(2) ** e < 1:
        e -= 1
    m = a / Fraction(2) ** (e - 23)            # in [2^23, 2^24)
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sgn * Fraction(n) * Fraction(2) ** (e - 23)


def _round_half_away(v):
    a = abs(Fraction(v))
    n = a.numerator // a.denominator
    if a - n >= Fraction(1, 2):
        n += 1
    return n if v >= 0 else -n


def test_q8_1_division_is_correctly_rounded(oracle_lib):
    """Readings R1-R2: d32 = amax / 127 and q = roundf(x / d32), each one
    correctly rounded fp32 division.  The block below (amax = A) was chosen
    so that both reciprocal shortcuts give other codes: d32 taken as
    A * fl(1/127) is one ulp lower, and x * fl(1/d32) rounds across a
    half-integer.  The expected codes come from exact rational arithmetic."""
    A = 1.6125396490097046
    xs = [A, 0.08253155648708344, -0.33647480607032776, 0.5269322395324707,
          -0.5396293997764587, 0.0698343887925148, 0.03174290433526039, -0.057137228548526764]
    x = np.zeros((1, 32), np.float32)
    x[0, :len(xs)] = xs
    assert all(float(np.float32(v)) == v for v in xs)
    d32 = _rne32(Fraction(A) / 127)
    exp = [_round_half_away(_rne32(Fraction(v) / d32)) for v in xs]
    # the shortcuts' codes differ (so a shortcut in the oracle would fail here)
    d_rcp = _rne32(Fraction(A) * _rne32(Fraction(1, 127)))
    q_rcp = [_round_half_away(_rne32(Fraction(v) * _rne32(1 / d32))) for v in xs]
    q_drcp = [_round_half_away(_rne32(Fraction(v) / d_rcp)) for v in xs]
    assert d_rcp != d32 and q_rcp != exp and q_drcp != exp
    assert exp[:7] == [127, 6, -26, 41, -42, 5, 2]
    D, S, q = _q8_fields(oracle_lib.quantize_q8_1(x), 1, 32)
    assert list(q[0, 0, :len(xs)]) == exp
    assert not q[0, 0, len(xs):].any()
    assert D[0, 0] == float(np.float16(float(d32)))
    assert Fraction(S[0, 0]) == Fraction(float(np.float16(float(Fraction(D[0, 0]) * sum(exp)))))


def test_q8_1_dequant_is_d_times_q(oracle_lib):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 512)).astype(np.float32)
    xq = oracle_lib.quantize_q8_1(x)
    D, S, q = _q8_fields(xq, 2, 512)
    xhat = oracle_lib.dequant_q8_1(xq, 2, 512)
    assert np.array_equal(xhat, (D[:, :, None] * q).reshape(2, 512))
    # reconstruction error bounded by half a step of the unrounded d32 plus the
    # binary16 rounding of d (relative 2^-11) times |q| <= 127
    d32 = np.abs(x.reshape(2, 16, 32)).max(axis=2) / 127.0
    bound = d32[:, :, None] * (0.5 + 127 * 2.0 ** -11) * 1.0001
    assert np.all(np.abs(x.reshape(2, 16, 32) - xhat.reshape(2, 16, 32)) <= bound)


# --------------------------------------------------------- weight decoders
def test_codebook_is_documented_placeholder(oracle_lib):
    cb = list(oracle_lib.codebook())
    assert cb == qf.placeholder_codebook()
    assert all(cb[i] < cb[i + 1] for i in range(15)) and max(abs(v) for v in cb) <= 127
    assert len(set(np.diff(cb))) > 1          # non-uniform


@pytest.mark.parametrize("wtype", TYPES)
def test_decoder_against_encoder(oracle_lib, wtype):
    rng = np.random.default_rng(100 + wtype)
    N, K = 3, 512
    fields = [[qf.random_fields(wtype, rng) for _ in range(K // 256)] for _ in range(N)]
    W = np.frombuffer(b"".join(qf.encode(wtype, f) for row in fields for f in row), dtype=np.uint8)
    got = oracle_lib.dequant(W, wtype, N, K)
    for n in range(N):
        for b in range(K // 256):
            exp = qf.dequant_exact(wtype, fields[n][b])
            seg = got[n, 256 * b:256 * (b + 1)]
            assert all(Fraction(float(seg[e])) == exp[e] for e in range(256)), (wtype, n, b)


@pytest.mark.parametrize("wtype", TYPES)
def test_decoder_single_bit_positions(oracle_lib, wtype):
    """Every code position, one at a time: the dequantized matrix must show the
    change at exactly the element the layout reading names."""
    rng = np.random.default_rng(7)
    base = qf.random_fields(wtype, rng)
    if wtype == qf.Q4_K:
        base["q"] = [0] * 256
        key, val = "q", 9
    elif wtype == qf.Q6_K:
        base["code"] = [-32] * 256
        base["sc"] = [int(v) or 1 for v in base["sc"]]
        key, val = "code", 21
    elif wtype in (qf.Q4_0, qf.Q8_0):
        base["d"] = [v if v & 0x7FFF else 0x3C00 for v in base["d"]]
        base["q"] = [0] * 256
        key, val = "q", 9 if wtype == qf.Q4_0 else 77
    else:
        base["idx"] = [0] * 256
        base["ls"] = [v if v != 32 else 33 for v in base["ls"]]
        key, val = "idx", 13
    ref = oracle_lib.dequant(np.frombuffer(qf.encode(wtype, base), np.uint8), wtype, 1, 256)[0]
    for e in range(256):
        f = dict(base)
        f[key] = list(base[key])
        f[key][e] = val
        got = oracle_lib.dequant(np.frombuffer(qf.encode(wtype, f), np.uint8), wtype, 1, 256)[0]
        changed = np.nonzero(got != ref)[0]
        assert list(changed) == [e], (wtype, e, changed[:4])


# ------------------------------------------------------------ matmul pins
def _build(wtype, rng, N, K, M):
    wf = [[qf.random_fields(wtype, rng) for _ in range(K // 256)] for _ in range(N)]
    xf = [qf.random_q8_fields(rng, K // 32) for _ in range(M)]
    W = np.frombuffer(b"".join(qf.encode(wtype, f) for row in wf for f in row), dtype=np.uint8)
    X = np.frombuffer(b"".join(qf.encode_q8(row) for row in xf), dtype=np.uint8)
    return wf, xf, W, X


@pytest.mark.parametrize("wtype", TYPES)
@pytest.mark.parametrize("N,K,M", [(1, 256, 1), (3, 512, 2), (4, 256, 3)])
def test_matmul_exact_rationals(oracle_lib, wtype, N, K, M):
    rng = np.random.default_rng(1000 * wtype + 10 * N + M)
    wf, xf, W, X = _build(wtype, rng, N, K, M)
    y_ex, is_ex = qf.exact_matmul(wtype, wf, xf, N, K, M)
    y64, ab, y32 = oracle_lib.qmatmul(W, wtype, N, K, X, M)
    isums = oracle_lib.isums(W, wtype, N, K, X, M)
    assert isums.tolist() == is_ex
    for m in range(M):
        for n in range(N):
            ex = y_ex[m][n]
            # fp64 summation of exact terms: error <= (#terms) * 2^-53 * sum|terms|
            assert abs(Fraction(float(y64[m, n])) - ex) <= Fraction(2 * K // 16 + 2, 2 ** 53) * Fraction(float(ab[m, n]))
            assert y32[m, n] == np.float32(y64[m, n])


@pytest.mark.parametrize("wtype", TYPES)
def test_matmul_equals_dequant_dot_when_s_is_consistent(oracle_lib, wtype):
    """Textbook identity: with Q8_1 blocks from the quantizer, S = D*sum(q) up to
    one binary16 rounding, and y = W_deq @ xhat - sum dmin*m*(S - D*sum q).
    Q6_K and IQ4_XS have no min term, so y is exactly dequantize-then-dot."""
    rng = np.random.default_rng(77 + wtype)
    N, K, M = 16, 1024, 3
    wf = [[qf.random_fields(wtype, rng) for _ in range(K // 256)] for _ in range(N)]
    W = np.frombuffer(b"".join(qf.encode(wtype, f) for row in wf for f in row), dtype=np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    X = oracle_lib.quantize_q8_1(x)
    xhat = oracle_lib.dequant_q8_1(X, M, K)
    wdeq = np.array([[float(v) for b in range(K // 256) for v in qf.dequant_exact(wtype, wf[n][b])]
                     for n in range(N)])
    ref = xhat @ wdeq.T
    if wtype == qf.Q4_K:
        D, S, q = _q8_fields(X, M, K)
        corr = np.zeros((M, N))
        for n in range(N):
            for b in range(K // 256):
                f = wf[n][b]
                dmin = float(qf.f16_frac(f["dmin"]))
                for j in range(8):
                    blk = 8 * b + j
                    corr[:, n] += dmin * f["mn"][j] * (S[:, blk] - D[:, blk] * q[:, blk].sum(axis=1))
        ref = ref - corr
    y64, ab, _ = oracle_lib.qmatmul(W, wtype, N, K, X, M)
    assert np.all(np.abs(y64 - ref) <= 1e-13 * ab + 1e-300)


@pytest.mark.parametrize("wtype", TYPES)
def test_one_hot_closed_form(oracle_lib, wtype):
    """x = v*e_k with v = 127*2^-6: D = 2^-6, q_k = 127, S = D*127 exactly and
    every other block is zero, so y[n] = (127/64) * w_deq[n, k] exactly."""
    rng = np.random.default_rng(3)
    N, K = 5, 512
    wf = [[qf.random_fields(wtype, rng) for _ in range(K // 256)] for _ in range(N)]
    W = np.frombuffer(b"".join(qf.encode(wtype, f) for row in wf for f in row), dtype=np.uint8)
    for k in (0, 1, 15, 16, 31, 32, 63, 64, 127, 128, 255, 256, 300, 511):
        x = np.zeros((1, K), dtype=np.float32)
        x[0, k] = 127 * 2.0 ** -6
        X = oracle_lib.quantize_q8_1(x)
        y64, _, _ = oracle_lib.qmatmul(W, wtype, N, K, X, 1)
        for n in range(N):
            wdeq = qf.dequant_exact(wtype, wf[n][k // 256])[k % 256]
            assert Fraction(float(y64[0, n])) == Fraction(127, 64) * wdeq, (wtype, k, n)


def test_special_cases(oracle_lib):
    rng = np.random.default_rng(9)
    K = 512
    # zero activations -> exactly zero
    for wtype in TYPES:
        wf, xf, W, X = _build(wtype, rng, 2, K, 1)
        X0 = oracle_lib.quantize_q8_1(np.zeros((1, K), np.float32))
        y64, _, _ = oracle_lib.qmatmul(W, wtype, 2, K, X0, 1)
        assert not y64.any()
    # Q4_K with all codes zero -> y = -sum dmin*m*S
    wf, xf, W, X = _build(qf.Q4_K, rng, 1, K, 1)
    for f in wf[0]:
        f["q"] = [0] * 256
    W = np.frombuffer(b"".join(qf.encode(qf.Q4_K, f) for f in wf[0]), np.uint8)
    y64, _, _ = oracle_lib.qmatmul(W, qf.Q4_K, 1, K, X, 1)
    exp = -sum(qf.f16_frac(wf[0][b]["dmin"]) * wf[0][b]["mn"][j] * qf.f16_frac(xf[0][8 * b + j][1])
               for b in range(2) for j in range(8))
    assert abs(Fraction(float(y64[0, 0])) - exp) <= abs(exp) * Fraction(1, 2 ** 48)
    # IQ4_XS ls = 32 and Q6_K sc = 0 zero a sub-block
    wf, xf, W, X = _build(qf.IQ4_XS, rng, 1, 256, 1)
    wf[0][0]["ls"] = [32] * 8
    W = np.frombuffer(qf.encode(qf.IQ4_XS, wf[0][0]), np.uint8)
    assert not oracle_lib.qmatmul(W, qf.IQ4_XS, 1, 256, X, 1)[0].any()
    wf, xf, W, X = _build(qf.Q6_K, rng, 1, 256, 1)
    wf[0][0]["sc"] = [0] * 16
    W = np.frombuffer(qf.encode(qf.Q6_K, wf[0][0]), np.uint8)
    assert not oracle_lib.qmatmul(W, qf.Q6_K, 1, 256, X, 1)[0].any()
    # Q4_0 nibbles all 8 (value q - 8 = 0) and Q8_0 codes all 0 give exactly 0
    for wtype, zero in ((qf.Q4_0, 8), (qf.Q8_0, 0)):
        wf, xf, W, X = _build(wtype, rng, 1, 256, 1)
        wf[0][0]["q"] = [zero] * 256
        W = np.frombuffer(qf.encode(wtype, wf[0][0]), np.uint8)
        assert not oracle_lib.qmatmul(W, wtype, 1, 256, X, 1)[0].any()
    # Q4_0 nibbles all 0 and 15: codes -8 and +7 times each block's d
    wf, xf, W, X = _build(qf.Q4_0, rng, 1, 256, 1)
    for nib, code in ((0, -8), (15, 7)):
        wf[0][0]["q"] = [nib] * 256
        W = np.frombuffer(qf.encode(qf.Q4_0, wf[0][0]), np.uint8)
        y64 = oracle_lib.qmatmul(W, qf.Q4_0, 1, 256, X, 1)[0][0, 0]
        exp = sum(qf.f16_frac(wf[0][0]["d"][j]) * code * qf.f16_frac(xf[0][j][0]) * sum(xf[0][j][2])
                  for j in range(8))
        assert abs(Fraction(float(y64)) - exp) <= abs(exp) * Fraction(1, 2 ** 48) + Fraction(1, 2 ** 200)


def test_rows_subset_matches_full(oracle_lib):
    from quant_integer_dot_amd import synth
    W = synth.weights(synth.Q6_K, 40, 512, (1, 2, 3))
    X = oracle_lib.quantize_q8_1(synth.activations(3, 512, (4, 5)))
    y64, ab, _ = oracle_lib.qmatmul(W, synth.Q6_K, 40, 512, X, 3)
    rows = np.array([0, 7, 39, 12])
    ys, abs_ = oracle_lib.qmatmul_rows(W, synth.Q6_K, 40, 512, X, 3, rows)
    assert np.array_equal(ys, y64[:, rows]) and np.array_equal(abs_, ab[:, rows])


def test_bad_arguments_rejected(oracle_lib):
    import ctypes
    W = np.zeros(144, np.uint8)
    X = np.zeros(36 * 8, np.uint8)
    y = np.zeros(4, np.float64)
    L = oracle_lib.lib()
    P = lambda a: ctypes.c_void_p(a.ctypes.data)
    assert L.oracle_qmatmul(P(W), 7, 1, 256, P(X), 1, P(y), None, None) == -1      # type
    assert L.oracle_qmatmul(P(W), 1, 1, 128, P(X), 1, P(y), None, None) == -1      # K % 256
    assert L.oracle_qmatmul(P(W), 1, 0, 256, P(X), 1, P(y), None, None) == -1      # N
    assert L.oracle_qmatmul(P(W), 1, 1, 256, P(X), 0, P(y), None, None) == -1      # M


# ------------------------------------------------- the pages' noise anchor
@pytest.mark.parametrize("wtype", TYPES)
def test_activation_quantization_noise_matches_pages(oracle_lib, wtype):
    """About 0.5 % RMS against fp32 SGEMV and the argmax kept (xLLM page B1.3)."""
    from quant_integer_dot_amd import synth
    g = json.load(open(os.path.join(GOLDEN, "q8_activation_noise.json")))
    N, K, M = 512, 4096, 2
    W = synth.weights(wtype, N, K, (2026, 99, wtype, 0))
    x = synth.activations(M, K, (2026, 99, K, M, 7))
    X = oracle_lib.quantize_q8_1(x)
    y64, _, _ = oracle_lib.qmatmul(W, wtype, N, K, X, M)
    wdeq = oracle_lib.dequant(W, wtype, N, K).astype(np.float32)
    ref = (x @ wdeq.T).astype(np.float64)                  # fp32 SGEMV
    rel = np.sqrt(np.mean((y64 - ref) ** 2) / np.mean(ref ** 2))
    lo, hi = g["test_band"]
    assert lo <= rel <= hi, rel
    # argmax kept whenever the fp32 top-2 gap exceeds 6x the predicted noise
    for m in range(M):
        top = np.argsort(ref[m])[::-1]
        gap = ref[m, top[0]] - ref[m, top[1]]
        if gap > 6 * rel * np.sqrt(np.mean(ref[m] ** 2)):
            assert int(np.argmax(y64[m])) == int(top[0])


# ------------------------------------------------ RMSNorm (fused producer)
# Pins of oracle.rmsnorm: a closed form, exact scale invariances, the fp64
# textbook formula within the fp32 error bound, and the page's summation
# order on a row worked out by hand where other orders give other fp32 sums.
def test_rmsnorm_constant_row_is_exactly_unit(oracle_lib):
    """x = c (a power of two), w = 1, eps = 0: mean = c^2, r = 1/|c| exactly,
    so every output is +-1 and the quantized block is the closed form."""
    K = 512
    for c in (2.0 ** -3, -4.0, 1.0):
        x = np.full((1, K), c, np.float32)
        xn, ss = oracle_lib.rmsnorm(x, np.ones(K, np.float32), 0.0)
        assert ss[0] == np.float32(K * c * c)
        assert np.all(xn == np.float32(np.sign(c)))
        xq = oracle_lib.rmsnorm_quantize_q8_1(x, np.ones(K, np.float32), 0.0).reshape(K // 32, 36)
        d32 = np.float32(1.0) / np.float32(127.0)
        assert np.all(xq[:, 4:].view(np.int8) == int(np.sign(c)) * 127)
        D = np.float16(d32)
        assert np.all(xq[:, 0:2].copy().view(np.float16) == D)


def test_rmsnorm_power_of_two_scale_invariance(oracle_lib):
    """Scaling x by 4 scales every square and sum by 16 and r by 1/4 exactly
    (eps = 0), so outputs and bytes are identical; scaling w by 2 doubles
    every output exactly."""
    rng = np.random.default_rng(11)
    M, K = 3, 1536
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    xn, _ = oracle_lib.rmsnorm(x, w, 0.0)
    xn4, _ = oracle_lib.rmsnorm(4 * x, w, 0.0)
    assert np.array_equal(xn.view(np.uint32), xn4.view(np.uint32))
    xn2, _ = oracle_lib.rmsnorm(x, 2 * w, 0.0)
    assert np.array_equal((2 * xn).view(np.uint32), xn2.view(np.uint32))
    assert np.array_equal(oracle_lib.rmsnorm_quantize_q8_1(x, w, 0.0),
                          oracle_lib.rmsnorm_quantize_q8_1(4 * x, w, 0.0))


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rmsnorm_matches_fp64_formula(oracle_lib, eps):
    """Against x / sqrt(mean(x^2) + eps) * w in fp64: a handful of fp32
    roundings, so within 8 units of 2^-24 relative (catches a missing 1/K,
    eps outside the root, an rsqrt-style approximation, a dropped weight)."""
    rng = np.random.default_rng(12)
    M, K = 4, 4096
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, K).astype(np.float32)
    xn, ss = oracle_lib.rmsnorm(x, w, eps)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + eps) * w.astype(np.float64)
    assert np.all(np.abs(xn - ref) <= 8 * 2.0 ** -24 * np.abs(ref) + 1e-30)
    assert np.allclose(ss, (x64 ** 2).sum(axis=1), rtol=1e-6)


def test_rmsnorm_sum_of_squares_order(oracle_lib):
    """Kestrel_VLLM #18, section 3.6: each group of 8 squares is summed as
    (lo0 + lo1) + (lo2 + lo3), lo_k = s_k + s_(k+4), and the group sums are
    added left to right into one fp32 accumulator.  Row (K = 64): group 0 is
    [2^12, 1, 1, 1, 1, 1, 1, 1], groups 1..7 are [1, 0, ..., 0].
      group 0: lo0 = 2^24 + 1, a tie, rounds to the even 2^24; lo1..lo3 = 2;
               s01 = 2^24 + 2, s23 = 4, group = 2^24 + 6 (all exact);
      groups 1..7: 1 each.
      serial:  (2^24 + 6) + 1 = 2^24 + 7, a tie between 2^24 + 6 (odd
               significand) and 2^24 + 8 (even): 2^24 + 8; every further + 1
               is a tie that rounds back to 2^24 + 8.  ss = 2^24 + 8.
    Other orders give other sums on this row (worked out the same way): the
    four groups of a 32-element block pairwise, then the blocks, gives
    2^24 + 14; one element at a time gives 2^24."""
    K = 64
    x = np.zeros((1, K), np.float32)
    x[0, 0:8] = [2.0 ** 12, 1, 1, 1, 1, 1, 1, 1]
    x[0, 8::8] = 1.0
    _, ss = oracle_lib.rmsnorm(x, np.ones(K, np.float32), 0.0)
    assert ss[0] == np.float32(2.0 ** 24 + 8)
    # the orders the page does not use give 2^24 + 14 and 2^24 on this row
    assert ss[0] != np.float32(2.0 ** 24 + 14) and ss[0] != np.float32(2.0 ** 24)
    # r and the outputs follow from ss: r = 1 / sqrt(ss / 64), x * r * 1
    r = np.float32(1.0) / np.sqrt(np.float32(ss[0] / np.float32(K)), dtype=np.float32)
    xn, _ = oracle_lib.rmsnorm(x, np.ones(K, np.float32), 0.0)
    assert np.array_equal(xn[0], (x[0] * r).astype(np.float32))


def test_rmsnorm_group_order_on_random_rows(oracle_lib):
    """The serial group order on ordinary rows: ss equals the group sums
    (each formed as the page's 8-wide horizontal sum) added left to right in
    numpy float32, for every row; the fp64 sum of squares is within K*2^-24
    relative of it."""
    rng = np.random.default_rng(13)
    M, K = 6, 4096
    x = rng.standard_normal((M, K)).astype(np.float32)
    _, ss = oracle_lib.rmsnorm(x, np.ones(K, np.float32), 1e-6)
    sq = (x * x).astype(np.float32).reshape(M, K // 8, 8)
    lo = (sq[:, :, 0:4] + sq[:, :, 4:8]).astype(np.float32)
    grp = ((lo[:, :, 0] + lo[:, :, 1]).astype(np.float32) + (lo[:, :, 2] + lo[:, :, 3]).astype(np.float32))
    for m in range(M):
        acc = np.float32(0.0)
        for g in grp[m].astype(np.float32):
            acc = np.float32(acc + g)
        assert ss[m] == acc, m
    ref = (x.astype(np.float64) ** 2).sum(axis=1)
    assert np.all(np.abs(ss - ref) <= K * 2.0 ** -24 * ref)


def test_rmsnorm_zero_row_quantizes_to_zero(oracle_lib):
    K = 256
    xq = oracle_lib.rmsnorm_quantize_q8_1(np.zeros((2, K), np.float32), np.ones(K, np.float32), 1e-6)
    assert not xq.any()
