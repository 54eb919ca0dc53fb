"""Test-side field encoders and exact rational evaluation.

These are the *inverse* of the oracle's decoders: they pack chosen field values
(scales, mins, codes, fp16 d) into superblock bytes following the written
layout readings, and evaluate the matmul definition on those field values with
Python Fractions.  A wrong index, shift or sign in the oracle's decoders or in
its arithmetic makes its output disagree with these.
"""
from fractions import Fraction

import numpy as np

Q4_K, Q6_K, IQ4_XS, Q4_0, Q8_0 = 1, 2, 3, 4, 5


def placeholder_codebook():
    """The documented stand-in codebook: round_half_away(-127 + 240*(i/15)**1.4)."""
    out = []
    for i in range(16):
        v = -127 + 240 * (i / 15) ** 1.4
        out.append(int(np.sign(v) * np.floor(abs(v) + 0.5)))
    return out


def f16_bits(x):
    return int(np.array([x], dtype=np.float16).view(np.uint16)[0])


def f16_frac(bits):
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def random_f16_bits(rng, scale=1e-3, allow_sub=True, signed=True):
    """fp16 bits of N(0, scale^2) (|N| when signed is False).  The workloads
    draw positive d and dmin, but the formats store them as signed binary16,
    so the pins feed both signs."""
    v = rng.standard_normal() * scale
    if not signed:
        v = abs(v)
    b = f16_bits(v)
    if not allow_sub and (b & 0x7C00) == 0:
        b |= 0x0400
    return b


# ------------------------------------------------------------------- Q4_K
def encode_q4_k(d, dmin, sc, mn, q):
    """d, dmin: fp16 bits; sc, mn: 8 ints in 0..63; q: 256 ints in 0..15."""
    b = bytearray(144)
    b[0:2] = d.to_bytes(2, "little")
    b[2:4] = dmin.to_bytes(2, "little")
    s = [0] * 12
    for j in range(4):
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        s[j + 4] = mn[j] | ((mn[j + 4] >> 4) << 6)
        s[j + 8] = (sc[j + 4] & 15) | ((mn[j + 4] & 15) << 4)
    b[4:16] = bytes(s)
    for c in range(4):
        for l in range(32):
            b[16 + 32 * c + l] = q[64 * c + l] | (q[64 * c + 32 + l] << 4)
    return bytes(b)


def q4_k_fields(rng):
    return dict(d=random_f16_bits(rng), dmin=random_f16_bits(rng),
                sc=[int(v) for v in rng.integers(0, 64, 8)],
                mn=[int(v) for v in rng.integers(0, 64, 8)],
                q=[int(v) for v in rng.integers(0, 16, 256)])


# ------------------------------------------------------------------- Q6_K
def encode_q6_k(d, sc, code):
    """d: fp16 bits; sc: 16 ints in -128..127; code: 256 ints in -32..31."""
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        u = code[e] + 32
        h, g, l = e // 128, (e % 128) // 32, e % 32
        ql[64 * h + 32 * (g & 1) + l] |= (u & 15) << (4 if g >= 2 else 0)
        qh[32 * h + l] |= (u >> 4) << (2 * g)
    b = bytearray(210)
    b[0:128] = bytes(ql)
    b[128:192] = bytes(qh)
    b[192:208] = bytes([v & 255 for v in sc])
    b[208:210] = d.to_bytes(2, "little")
    return bytes(b)


def q6_k_fields(rng):
    return dict(d=random_f16_bits(rng),
                sc=[int(v) for v in rng.integers(-128, 128, 16)],
                code=[int(v) for v in rng.integers(-32, 32, 256)])


# ----------------------------------------------------------------- IQ4_XS
def encode_iq4_xs(d, ls, idx):
    """d: fp16 bits; ls: 8 ints in 0..63; idx: 256 ints in 0..15."""
    b = bytearray(136)
    b[0:2] = d.to_bytes(2, "little")
    sh = 0
    sl = [0] * 4
    for j in range(8):
        sh |= ((ls[j] >> 4) & 3) << (2 * j)
        sl[j // 2] |= (ls[j] & 15) << (4 * (j % 2))
    b[2:4] = sh.to_bytes(2, "little")
    b[4:8] = bytes(sl)
    for j in range(8):
        for i in range(16):
            b[8 + 16 * j + i] = idx[32 * j + i] | (idx[32 * j + 16 + i] << 4)
    return bytes(b)


def iq4_xs_fields(rng):
    return dict(d=random_f16_bits(rng),
                ls=[int(v) for v in rng.integers(0, 64, 8)],
                idx=[int(v) for v in rng.integers(0, 16, 256)])


# ------------------------------------------------------ Q4_0 / Q8_0 (x 8)
# The fields of a 256-weight group: eight blocks of 32, each its own d.
def encode_q4_0(d, q):
    """d: 8 fp16 bits; q: 256 raw nibbles in 0..15 (value = d_j * (q - 8))."""
    b = bytearray()
    for j in range(8):
        b += d[j].to_bytes(2, "little")
        b += bytes(q[32 * j + i] | (q[32 * j + 16 + i] << 4) for i in range(16))
    return bytes(b)


def encode_q8_0(d, q):
    """d: 8 fp16 bits; q: 256 ints in -128..127 (value = d_j * q)."""
    b = bytearray()
    for j in range(8):
        b += d[j].to_bytes(2, "little") + bytes(v & 255 for v in q[32 * j:32 * j + 32])
    return bytes(b)


def q4_0_fields(rng):
    return dict(d=[random_f16_bits(rng) for _ in range(8)],
                q=[int(v) for v in rng.integers(0, 16, 256)])


def q8_0_fields(rng):
    return dict(d=[random_f16_bits(rng) for _ in range(8)],
                q=[int(v) for v in rng.integers(-128, 128, 256)])


# --------------------------------------------------------- generic helpers
def random_fields(wtype, rng):
    return {Q4_K: q4_k_fields, Q6_K: q6_k_fields, IQ4_XS: iq4_xs_fields,
            Q4_0: q4_0_fields, Q8_0: q8_0_fields}[wtype](rng)


def encode(wtype, f):
    if wtype == Q4_K:
        return encode_q4_k(f["d"], f["dmin"], f["sc"], f["mn"], f["q"])
    if wtype == Q6_K:
        return encode_q6_k(f["d"], f["sc"], f["code"])
    if wtype == Q4_0:
        return encode_q4_0(f["d"], f["q"])
    if wtype == Q8_0:
        return encode_q8_0(f["d"], f["q"])
    return encode_iq4_xs(f["d"], f["ls"], f["idx"])


def sublen(wtype):
    return 16 if wtype == Q6_K else 32


def codes_and_scales(wtype, f):
    """(codes[256], per-sub-block (scale Fraction, min Fraction))."""
    if wtype == Q4_K:
        d, dmin = f16_frac(f["d"]), f16_frac(f["dmin"])
        return list(f["q"]), [(d * f["sc"][j], dmin * f["mn"][j]) for j in range(8)]
    if wtype == Q6_K:
        d = f16_frac(f["d"])
        return list(f["code"]), [(d * f["sc"][t], Fraction(0)) for t in range(16)]
    if wtype == Q4_0:
        return [v - 8 for v in f["q"]], [(f16_frac(f["d"][j]), Fraction(0)) for j in range(8)]
    if wtype == Q8_0:
        return list(f["q"]), [(f16_frac(f["d"][j]), Fraction(0)) for j in range(8)]
    cb = placeholder_codebook()
    d = f16_frac(f["d"])
    return [cb[i] for i in f["idx"]], [(d * (f["ls"][j] - 32), Fraction(0)) for j in range(8)]


def dequant_exact(wtype, f):
    codes, sm = codes_and_scales(wtype, f)
    L = sublen(wtype)
    return [sm[e // L][0] * codes[e] - sm[e // L][1] for e in range(256)]


def random_q8_fields(rng, nblk, sub_ok=True):
    """Arbitrary Q8_1 blocks: (D bits, S bits, q[32]) each; S independent of q."""
    out = []
    for _ in range(nblk):
        D = random_f16_bits(rng, scale=0.02)
        S = f16_bits(rng.standard_normal() * 2.0)
        q = [int(v) for v in rng.integers(-127, 128, 32)]
        out.append((D, S, q))
    return out


def encode_q8(blocks):
    b = bytearray()
    for D, S, q in blocks:
        b += D.to_bytes(2, "little") + S.to_bytes(2, "little") + bytes([v & 255 for v in q])
    return bytes(b)


def exact_matmul(wtype, wfields, xblocks, N, K, M):
    """Exact y[m][n] (Fractions), exact isums[m][n][sub], from field values.

    wfields[n][b] are per-superblock field dicts; xblocks[m][k/32] are Q8_1
    field triples."""
    L = sublen(wtype)
    nsb = K // 256
    y = [[Fraction(0)] * N for _ in range(M)]
    isum = [[[0] * (K // L) for _ in range(N)] for _ in range(M)]
    for n in range(N):
        for b in range(nsb):
            codes, sm = codes_and_scales(wtype, wfields[n][b])
            for m in range(M):
                for j in range(256 // L):
                    k0 = 256 * b + L * j
                    D, S, q = xblocks[m][k0 // 32]
                    I = sum(codes[L * j + i] * q[(k0 + i) % 32] for i in range(L))
                    isum[m][n][(256 // L) * b + j] = I
                    y[m][n] += sm[j][0] * f16_frac(D) * I - sm[j][1] * f16_frac(S)
    return y, isum
