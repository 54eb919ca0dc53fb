"""Seeded synthetic inputs: raw weight superblocks and fp32 activations.

This module is shared by the tests, the benchmark and the smoke check.  It holds
none of the matmul's arithmetic: it only draws random bytes and writes the
stated value distributions into the fields of each superblock.

Distributions (the workloads of the xLLM and V100TPS pages are GGUF checkpoints
of Qwen2.5-1.5B, Qwen3-8B and a hidden-5120 IQ4_XS model; their trained
weights are not available, so seeded inputs of the same shapes stand in):
  * Q4_K  : quant and scale bytes uniform random (nibbles uniform 0..15, 6-bit
            scales and mins uniform 0..63); d, dmin ~ |N(0, 1e-3)| as binary16.
  * Q6_K  : ql, qh bytes uniform random; 16 int8 sub-scales round(N(0, 30))
            clipped to [-128, 127]; d ~ |N(0, 1e-3)| as binary16.
  * IQ4_XS: index, scales_h and scales_l bytes uniform random (indices 0..15,
            6-bit scales 0..63); d ~ |N(0, 1e-3)| as binary16.
  * Q4_0 / Q8_0: per 32-weight block, quant bytes uniform random (nibbles
            0..15, int8 codes -128..127) and d ~ |N(0, 1e-3)| as binary16;
            eight blocks make up each 256-weight group.
  * activations: fp32 N(0, 1).
Seeds: numpy SeedSequence([2026, config, layer, projection]) for weights and
SeedSequence([2026, config, K, M, 7]) for activations.
"""
import numpy as np

Q4_K, Q6_K, IQ4_XS, Q4_0, Q8_0 = 1, 2, 3, 4, 5
TYPE_NAMES = {Q4_K: "Q4_K", Q6_K: "Q6_K", IQ4_XS: "IQ4_XS", Q4_0: "Q4_0", Q8_0: "Q8_0"}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, IQ4_XS: 136, Q4_0: 144, Q8_0: 272}   # per 256 weights

# (name, N, K, type) per projection; N = output rows, K = input width.
QWEN25_1P5B = [
    ("q", 1536, 1536, Q4_K), ("k", 256, 1536, Q4_K), ("v", 256, 1536, Q4_K),
    ("o", 1536, 1536, Q4_K), ("gate", 8960, 1536, Q4_K), ("up", 8960, 1536, Q4_K),
    ("down", 1536, 8960, Q4_K),
]
QWEN3_8B = [
    ("q", 4096, 4096, Q4_K), ("k", 1024, 4096, Q4_K), ("v", 1024, 4096, Q6_K),
    ("o", 4096, 4096, Q4_K), ("gate", 12288, 4096, Q4_K), ("up", 12288, 4096, Q4_K),
    ("down", 4096, 12288, Q6_K),
]
# The same shapes in the simple block formats: Q4_0 where the mixed model has
# Q4_K, Q8_0 where it has Q6_K.
QWEN3_8B_Q40_Q80 = [(n, N, K, Q4_0 if t == Q4_K else Q8_0) for (n, N, K, t) in QWEN3_8B]
IQ4XS_H5120 = [
    ("qkv", 7168, 5120, IQ4_XS), ("o", 5120, 5120, IQ4_XS),
    ("gate", 17408, 5120, IQ4_XS), ("up", 17408, 5120, IQ4_XS),
    ("down", 5120, 17408, IQ4_XS),
]
# One GPU's share of the Qwen3-8B layer under 8-way tensor parallelism:
# q, k, v, gate and up split by output rows (column-parallel), o and down by
# K (row-parallel, whole superblocks: 4096 / 8 = 512 and 12288 / 8 = 1536).
QWEN3_8B_TP8 = [
    ("q", 512, 4096, Q4_K), ("k", 128, 4096, Q4_K), ("v", 128, 4096, Q6_K),
    ("o", 4096, 512, Q4_K), ("gate", 1536, 4096, Q4_K), ("up", 1536, 4096, Q4_K),
    ("down", 4096, 1536, Q6_K),
]

# Workloads: index -> description.  Index 4 reuses the Qwen3-8B shapes at M=512.
WORKLOADS = {
    0: dict(name="q4k-matvec-1536", shapes=[("w", 1536, 1536, Q4_K)], layers=1, Ms=[1]),
    1: dict(name="qwen2.5-1.5b-decode", shapes=QWEN25_1P5B, layers=28, Ms=[1, 2, 4, 8]),
    2: dict(name="qwen3-8b-decode", shapes=QWEN3_8B, layers=36, Ms=list(range(1, 9))),
    3: dict(name="iq4xs-h5120-decode", shapes=IQ4XS_H5120, layers=64, Ms=list(range(1, 9))),
    4: dict(name="qwen3-8b-prefill-512", shapes=QWEN3_8B, layers=36, Ms=[512]),
    5: dict(name="qwen3-8b-q4_0-q8_0-decode", shapes=QWEN3_8B_Q40_Q80, layers=36, Ms=[1, 2, 4, 8]),
    6: dict(name="qwen3-8b-mid-batch", shapes=QWEN3_8B, layers=36, Ms=[16, 32, 64, 96]),
    7: dict(name="qwen3-8b-tp8-shard-decode", shapes=QWEN3_8B_TP8, layers=36, Ms=list(range(1, 9))),
}


def rng_for(*seed):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(s) for s in seed])))


def _half_bytes(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32).astype(np.float16)).view(np.uint8)


def weight_bytes(wtype, N, K):
    return N * (K // 256) * BLOCK_BYTES[wtype]


def weights(wtype, N, K, seed, signed_scales=False):
    """Raw superblocks, uint8 [N][K/256 * block_bytes] (GGUF row order).

    signed_scales: give every fp16 d (and Q4_K dmin) a random sign.  The
    workloads draw them positive; the formats store signed binary16, and the
    parity tests cover both signs."""
    assert K % 256 == 0 and N >= 1
    rng = rng_for(*seed)
    nb = K // 256
    B = BLOCK_BYTES[wtype]
    raw = np.frombuffer(rng.bytes(N * nb * B), dtype=np.uint8).reshape(N, nb, B).copy()
    d = np.abs(rng.standard_normal((N, nb)) * 1e-3)
    if signed_scales:
        d = d * rng.choice([-1.0, 1.0], size=d.shape)
    if wtype == Q4_K:
        dmin = np.abs(rng.standard_normal((N, nb)) * 1e-3)
        if signed_scales:
            dmin = dmin * rng.choice([-1.0, 1.0], size=dmin.shape)
        raw[:, :, 0:2] = _half_bytes(d).reshape(N, nb, 2)
        raw[:, :, 2:4] = _half_bytes(dmin).reshape(N, nb, 2)
    elif wtype == Q6_K:
        sc = np.clip(np.rint(rng.standard_normal((N, nb, 16)) * 30.0), -128, 127).astype(np.int8)
        raw[:, :, 192:208] = sc.view(np.uint8)
        raw[:, :, 208:210] = _half_bytes(d).reshape(N, nb, 2)
    elif wtype == IQ4_XS:
        raw[:, :, 0:2] = _half_bytes(d).reshape(N, nb, 2)
    elif wtype in (Q4_0, Q8_0):
        bb = B // 8
        dj = np.abs(rng.standard_normal((N, nb, 8)) * 1e-3)
        if signed_scales:
            dj = dj * rng.choice([-1.0, 1.0], size=dj.shape)
        blk = raw.reshape(N, nb, 8, bb)
        blk[:, :, :, 0:2] = _half_bytes(dj).reshape(N, nb, 8, 2)
    else:
        raise ValueError(f"unknown weight type {wtype}")
    return raw.reshape(N, nb * B)


def kv4_row_bytes(D):
    """Bytes of one K or V row of D elements in the 4-bit KV cache."""
    return D // 32 * 18


def kv4_cache(Hkv, T, D, seed, dscale=0.08):
    """4-bit KV cache, uint8 [Hkv][T][D/32 * 18]: per row D/32 blocks of an
    fp16 scale d ~ |N(0, dscale^2)| + dscale/4 and 16 bytes of random
    nibbles (values d * (q - 8), so elements up to about +-1 as in a model's
    K and V)."""
    assert D % 32 == 0 and T >= 1 and Hkv >= 1
    rng = rng_for(*seed)
    nb = D // 32
    raw = np.frombuffer(rng.bytes(Hkv * T * nb * 18), dtype=np.uint8).reshape(Hkv, T, nb, 18).copy()
    d = np.abs(rng.standard_normal((Hkv, T, nb))) * dscale + dscale / 4
    raw[:, :, :, 0:2] = _half_bytes(d).reshape(Hkv, T, nb, 2)
    return raw.reshape(Hkv, T, nb * 18)


def activations(M, K, seed):
    """fp32 [M][K] ~ N(0, 1)."""
    rng = rng_for(*seed)
    return rng.standard_normal((M, K), dtype=np.float32)


def weight_seed(config, layer, proj):
    return (2026, config, layer, proj)


def act_seed(config, K, M):
    return (2026, config, K, M, 7)
