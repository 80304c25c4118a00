"""Seeded synthetic inputs (numpy, PCG64).

This module only draws numbers: activations, dense weights, 4-bit codes,
scales and biases, as bf16 bit patterns, binary32 values or bytes.  It
contains none of the sharded-linear arithmetic and is the one piece of code
that both the GPU path's tests and the CPU oracle consume (as input bytes).

Seeds are derived from (config, projection, tensor, variant) so that every
tensor of every workload is reproducible on its own:
    seed = 100000 * config + 1000 * projection + 10 * tensor + variant
with tensor ids X=1, W=2, codes=3, scales=4, biases=5 and variant 0 for the
random draw, 1 for the small-integer draw.
"""
import numpy as np

T_X, T_W, T_CODES, T_SCALES, T_BIASES = 1, 2, 3, 4, 5


def seed_of(config, proj, tensor, variant=0):
    return 100000 * int(config) + 1000 * int(proj) + 10 * int(tensor) + int(variant)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x):
    """Round binary32 values to bf16 (nearest, ties to even): uint16 bits.

    Used only to draw bf16-valued inputs; NaN is not expected here.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = (b + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bf16 bit patterns to binary32 (for building inputs)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed, shape, std=1.0):
    return (rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def normal_bf16(seed, shape, std=1.0):
    """bf16 bit patterns of N(0, std^2) draws."""
    return f32_to_bf16_bits(normal_f32(seed, shape, std))


def small_int(seed, shape, lo=-3, hi=3):
    """Integers uniform on {lo..hi} as binary32 values."""
    return rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def small_int_bf16(seed, shape, lo=-3, hi=3):
    return f32_to_bf16_bits(small_int(seed, shape, lo, hi))


def q4_codes(seed, shape):
    """4-bit codes uniform on 0..15, one byte each."""
    return rng(seed).integers(0, 16, size=shape, dtype=np.uint8)


def uniform_bf16(seed, shape, lo, hi):
    return f32_to_bf16_bits(rng(seed).uniform(lo, hi, size=shape).astype(np.float32))


def const_bf16(shape, value):
    return np.full(shape, f32_to_bf16_bits(np.float32(value)), dtype=np.uint16)


def token_ids(seed, M, vocab):
    """M token ids uniform on 0..vocab-1, int32."""
    return rng(seed).integers(0, vocab, size=M, dtype=np.int32)


def router(seed, T, k, n_experts):
    """Router outputs: each token's k distinct experts (uniform), int32
    [T][k], and their weights, a softmax of N(0, 1) logits over the k
    choices, binary32 [T][k]."""
    g = rng(seed)
    topk = np.argsort(g.random((T, n_experts)), axis=1)[:, :k].astype(np.int32)
    logits = g.standard_normal((T, k))
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return topk, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def wide_rows_bf16(seed, M, K):
    """bf16 activations whose rows span the bf16 range: row m is N(0, 1)
    scaled by a pattern chosen by m % 7 -- 1e6; 1e-30; N(0, 1) with one
    element set to +-3e38; 2^U(-60, 60) per element; plain N(0, 1); 1e-39
    (bf16 subnormals); N(0, 1) with one element 65536 (just past binary16)."""
    g = rng(seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    kind = np.arange(M) % 7
    x[kind == 0] *= np.float32(1e6)
    x[kind == 1] *= np.float32(1e-30)
    big = np.nonzero(kind == 2)[0]
    x[big, g.integers(0, K, size=big.size)] = np.where(g.random(big.size) < 0.5, -3e38, 3e38)
    mixed = np.nonzero(kind == 3)[0]
    x[mixed] *= np.exp2(g.uniform(-60, 60, size=(mixed.size, K))).astype(np.float32)
    x[kind == 5] *= np.float32(1e-39)
    edge = np.nonzero(kind == 6)[0]
    x[edge, g.integers(0, K, size=edge.size)] = np.float32(65536.0)
    return f32_to_bf16_bits(x)


def wide_scales_bf16(seed, shape, lo=0.005, hi=0.02):
    """4-bit group scales U(lo, hi) times a per-column 10^U(-30, 30), and per
    group a further 2^U(-20, 20): columns and groups far apart in magnitude."""
    g = rng(seed)
    G, N = shape
    s = g.uniform(lo, hi, size=shape)
    s *= 10.0 ** g.uniform(-30, 30, size=(1, N))
    s *= np.exp2(g.uniform(-20, 20, size=shape))
    return f32_to_bf16_bits(s.astype(np.float32))


def wide_biases_bf16(seed, scales_bits, std=3.0):
    """Biases N(0, std^2) times the group's own scale (same magnitude class)."""
    s = bf16_bits_to_f32(scales_bits).astype(np.float64)
    b = rng(seed).standard_normal(s.shape) * std * s
    return f32_to_bf16_bits(b.astype(np.float32))


def big_int_rows_bf16(seed, M, K, top=20):
    """Integers in {-3..3} with one element per row replaced by +-2^j, j
    uniform on 0..top: integer-valued rows up to 2^top in magnitude."""
    g = rng(seed)
    x = g.integers(-3, 4, size=(M, K)).astype(np.float32)
    j = g.integers(0, top + 1, size=M)
    sign = np.where(g.random(M) < 0.5, -1.0, 1.0)
    x[np.arange(M), g.integers(0, K, size=M)] = (sign * np.exp2(j)).astype(np.float32)
    return f32_to_bf16_bits(x)
