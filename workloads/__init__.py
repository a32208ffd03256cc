"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and lays them out; it holds none of the
arithmetic of the method itself (no activation quantization, no integer dot
products, no epilogue, no tree, no argmax, no scale requantization).  Both
the tests and the benchmark take their inputs from here, so the oracle and
the HIP library always see the same bytes.

Recipes (numpy ``Generator(PCG64(seed))``; draws happen in the order listed):
  * int8 weights: ``integers(-127, 128)``, uniform on [-127, 127];
  * per-output-channel fp32 scales: log-uniform on [1e-3, 1e-1];
  * activations: ``standard_normal`` as fp32, rounded to bf16 (round to
    nearest even, by torch's CPU conversion);
  * outlier channels: ``round(0.01 * K)`` channel indices from a seeded
    permutation, the same for every token, scaled by 20 in fp32 and rounded
    to bf16 again;
  * FP8 (E4M3) weights, drawn as codes: sign uniform, exponent field
    ``rint(normal(12.5, 1.5))`` clipped to [0, 15], mantissa uniform on
    [0, 7], the NaN code (exponent 15, mantissa 7) replaced by the largest
    finite one, 0x7E; magnitudes then cluster a few octaves below 448, as for
    weights quantized per row at amax / 448.  Per-row fp32 scales
    log-uniform on [1e-5, 1e-3];
  * decode attention: q, k and v ``standard_normal`` rounded to bf16 (the
    post-norm, post-rotary statistics of a Qwen3 layer are of that order);
    cache slots past the cells in use hold NaN bit patterns (0x7FC0), so a
    kernel that reads past a query's position shows it in its output;
  * q8_0-style block weights: real weights ``standard_normal``, per aligned
    32-block an fp16 scale ``d = fp16(amax / 127)`` and int8 codes
    ``clamp(rint(w / d), -127, 127)`` (0 where d == 0).  This is the
    preparation of a weight file, not a step of the linear layer;
  * kq6 superblock weights (256 weights per superblock, this library's own
    layout): codes uniform on [-32, 31], int8 sub-scales (one per 16
    weights) uniform on [-127, 127], fp16 superblock scales log-uniform on
    [1e-6, 1e-4]; the codes are then laid out in the two bit planes;
  * kq4 superblock weights: codes uniform on [0, 15], per 32 weights a
    sub-scale and a minimum uniform on [0, 63], per superblock fp16 d
    log-uniform on [1e-5, 1e-3] and dmin log-uniform on [1e-4, 1e-2].

The layer shapes follow Qwen3 models (hidden size, intermediate size and the
packed qkv / gate_up projections); no model weights are used or needed.

bf16 and fp16 tensors are returned as their uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# -- shapes -------------------------------------------------------------------

# (name, K, N): input features K, output features N.
TINY = ("tiny", 512, 256)
QWEN3_8B = [("qkv", 4096, 6144), ("o", 4096, 4096), ("gate_up", 4096, 24576), ("down", 12288, 4096)]
QWEN3_14B = [("qkv", 5120, 7168), ("o", 5120, 5120), ("gate_up", 5120, 34816), ("down", 17408, 5120)]
BLOCKQ8_SHAPES = [("bq8_4096", 4096, 4096), ("bq8_12288", 12288, 4096)]
LM_HEAD = ("lm_head", 4096, 151936)
# decode attention: (name, query heads, kv heads, head dim)
QWEN3_8B_ATTN = ("qwen3_8b_attn", 32, 8, 128)

SEED_TINY = 1001
SEED_8B = 2001
SEED_BQ8 = 3001
SEED_14B = 4001
SEED_LM_HEAD = 5001
SEED_ATTN = 6001
SEED_FP8 = 7001

TOKENS_TINY = 5
TOKENS_8B = 512
TOKENS_BQ8 = 16
TOKENS_14B = 512
TOKENS_LM_HEAD = 64


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) with torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def int8_weights(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    return g.integers(-127, 128, size=(N, K), dtype=np.int8)


def log_uniform_scales(g: np.random.Generator, n: int, lo: float = 1e-3, hi: float = 1e-1) -> np.ndarray:
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=n)).astype(np.float32)


def normal_bf16(g: np.random.Generator, b: int, K: int) -> np.ndarray:
    return f32_to_bf16_bits(g.standard_normal(size=(b, K), dtype=np.float32))


def add_outlier_channels(g: np.random.Generator, x_bits: np.ndarray, frac: float = 0.01,
                         factor: float = 20.0) -> tuple[np.ndarray, np.ndarray]:
    """Scale round(frac*K) seeded channels by `factor` (fp32) and re-round to bf16."""
    K = x_bits.shape[1]
    n_out = int(round(frac * K))
    idx = np.sort(g.permutation(K)[:n_out])
    x = bf16_bits_to_f32(x_bits).copy()
    x[:, idx] = x[:, idx] * np.float32(factor)
    return f32_to_bf16_bits(x), idx


def q8_0_weights(g: np.random.Generator, N: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    """q8_0-style weight file: int8 codes [N, K] and fp16 block scales [N, K/32] (uint16 bits)."""
    assert K % 32 == 0
    w = g.standard_normal(size=(N, K // 32, 32), dtype=np.float32)
    amax = np.abs(w).max(axis=2)
    d16 = (amax / np.float32(127.0)).astype(np.float32).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    codes = np.rint(w / safe[:, :, None])
    codes = np.clip(codes, -127, 127)
    codes = np.where((d32 == 0)[:, :, None], 0, codes).astype(np.int8)
    return codes.reshape(N, K), d16.view(np.uint16).copy()


# -- whole-config generators -----------------------------------------------------

@dataclass
class W8A8Layer:
    name: str
    K: int
    N: int
    w: np.ndarray        # int8 [N, K]
    s_w: np.ndarray      # fp32 [N]
    x: np.ndarray        # bf16 bits [T, K]
    outliers: np.ndarray | None


def w8a8_layer(name: str, K: int, N: int, seed: int, tokens: int, outliers: bool) -> W8A8Layer:
    g = rng(seed)
    w = int8_weights(g, N, K)
    s_w = log_uniform_scales(g, N)
    x = normal_bf16(g, tokens, K)
    idx = None
    if outliers:
        x, idx = add_outlier_channels(g, x)
    return W8A8Layer(name, K, N, w, s_w, x, idx)


def tiny_layer() -> W8A8Layer:
    name, K, N = TINY
    return w8a8_layer(name, K, N, SEED_TINY, TOKENS_TINY, outliers=False)


def qwen3_8b_layer(i: int, tokens: int = TOKENS_8B) -> W8A8Layer:
    name, K, N = QWEN3_8B[i]
    return w8a8_layer(name, K, N, SEED_8B + i, tokens, outliers=True)


def qwen3_14b_layer(i: int, tokens: int = TOKENS_14B) -> W8A8Layer:
    name, K, N = QWEN3_14B[i]
    return w8a8_layer(name, K, N, SEED_14B + i, tokens, outliers=True)


def lm_head_layer(tokens: int = TOKENS_LM_HEAD) -> W8A8Layer:
    name, K, N = LM_HEAD
    return w8a8_layer(name, K, N, SEED_LM_HEAD, tokens, outliers=False)


@dataclass
class BlockQ8Layer:
    name: str
    K: int
    N: int
    w: np.ndarray        # int8 [N, K]
    d_w: np.ndarray      # fp16 bits [N, K/32]
    x: np.ndarray        # bf16 bits [T, K]


def blockq8_layer(i: int, tokens: int = TOKENS_BQ8) -> BlockQ8Layer:
    name, K, N = BLOCKQ8_SHAPES[i]
    g = rng(SEED_BQ8 + i)
    w, d_w = q8_0_weights(g, N, K)
    x = normal_bf16(g, tokens, K)
    return BlockQ8Layer(name, K, N, w, d_w, x)


# -- crafted inputs for the block tree ------------------------------------------

FP16_ONE = 0x3C00           # 1.0
FP16_2P15 = 0x7800          # 2^15


def tree_witness_operands(K: int, groups_per_row: list[list[tuple[int, int]]], b: int = 1):
    """Operands whose block partials are the leaf pattern [2^27, 1, -2^27, 1].

    Every block of the shared activations holds q = 1 at its first element and
    q = 64 at its second, with d_a = 1.  Row r of the weights places, for each
    (p, h) in groups_per_row[r], the four leaves at blocks p, p+h, p+2h, p+3h
    (p a multiple of 4h, so that the pattern spans one aligned subtree):
      2^27  : w = +64 at the second element, d_w = 2^15  (isum = 4096)
      1     : w = 1 at the first element,    d_w = 1     (isum = 1)
      -2^27 : w = -64 at the second element, d_w = 2^15
    Every other block of the row has w = 0 (a +0 leaf).

    Returns q int8 [b, K], d_a fp32 [b, K/32], w int8 [R, K], d_w fp16 bits [R, K/32].
    """
    m = K // 32
    R = len(groups_per_row)
    q = np.zeros((b, K), np.int8)
    q[:, 0::32] = 1
    q[:, 1::32] = 64
    d_a = np.ones((b, m), np.float32)
    w = np.zeros((R, K), np.int8)
    d_w = np.full((R, m), FP16_ONE, np.uint16)
    for r, groups in enumerate(groups_per_row):
        for p, h in groups:
            assert p % (4 * h) == 0 and p + 3 * h < m, (p, h, m)
            for j, kind in zip((p, p + h, p + 2 * h, p + 3 * h), ("big+", "one", "big-", "one")):
                if kind == "one":
                    w[r, 32 * j] = 1
                else:
                    w[r, 32 * j + 1] = 64 if kind == "big+" else -64
                    d_w[r, j] = FP16_2P15
    return q, d_a, w, d_w


def negative_zero_operands(K: int, N: int = 4, b: int = 1):
    """Operands whose every block partial is -0: all activation codes 0 and
    d_a = -1, weights and d_w arbitrary (here 1).  The sum of -0 leaves is -0;
    adding the +0 leaves of a zero-padded tree turns it into +0."""
    m = K // 32
    q = np.zeros((b, K), np.int8)
    d_a = np.full((b, m), -1.0, np.float32)
    w = np.ones((N, K), np.int8)
    d_w = np.full((N, m), FP16_ONE, np.uint16)
    return q, d_a, w, d_w


# -- decode attention ---------------------------------------------------------------

BF16_NAN = 0x7FC0


@dataclass
class AttnCase:
    q: np.ndarray        # bf16 bits [b, Hq, D]
    k: np.ndarray        # bf16 bits [capacity, Hkv, D]
    v: np.ndarray        # bf16 bits [capacity, Hkv, D]
    pos0: int            # query t sits at position pos0 + t
    scale: np.float32    # 1 / sqrt(D), rounded to binary32


def attn_case(seed: int, b: int, cells: int, Hq: int = 32, Hkv: int = 8, D: int = 128,
              capacity: int | None = None) -> AttnCase:
    """b queries at positions cells - b .. cells - 1 over a cache holding
    `cells` written cells (the queries' own keys included) in an allocation
    of `capacity` slots; slots past `cells` are NaN."""
    assert 1 <= b <= cells
    capacity = cells if capacity is None else capacity
    g = rng(seed)
    q = normal_bf16(g, b * Hq, D).reshape(b, Hq, D)
    k = np.full((capacity, Hkv, D), BF16_NAN, np.uint16)
    v = np.full((capacity, Hkv, D), BF16_NAN, np.uint16)
    k[:cells] = normal_bf16(g, cells * Hkv, D).reshape(cells, Hkv, D)
    v[:cells] = normal_bf16(g, cells * Hkv, D).reshape(cells, Hkv, D)
    return AttnCase(q, k, v, cells - b, np.float32(1.0 / np.sqrt(np.float64(D))))


# -- FP8 (E4M3) weights ------------------------------------------------------------

def e4m3_weight_codes(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    sign = g.integers(0, 2, (N, K)).astype(np.uint8)
    exp = np.clip(np.rint(g.normal(12.5, 1.5, (N, K))), 0, 15).astype(np.uint8)
    man = g.integers(0, 8, (N, K)).astype(np.uint8)
    codes = (sign << 7) | (exp << 3) | man
    nan = (codes & 0x7F) == 0x7F
    codes[nan] = (codes[nan] & 0x80) | 0x7E
    return codes


@dataclass
class FP8Layer:
    name: str
    K: int
    N: int
    w: np.ndarray        # e4m3 codes uint8 [N, K]
    s_w: np.ndarray      # fp32 [N]
    x: np.ndarray        # bf16 bits [T, K]


def fp8_layer(i: int, tokens: int = 16) -> FP8Layer:
    """Qwen3-8B-shaped layer i with FP8 weights; activations as the W8A8 layers."""
    name, K, N = QWEN3_8B[i]
    g = rng(SEED_FP8 + i)
    w = e4m3_weight_codes(g, N, K)
    s_w = log_uniform_scales(g, N, 1e-5, 1e-3)
    x = normal_bf16(g, tokens, K)
    x, _ = add_outlier_channels(g, x)
    return FP8Layer(name, K, N, w, s_w, x)


# -- kq6: k-quant-style superblocks of 256 weights with 6-bit codes ------------------
#
# Layout (this library's own; the pages give none): code c in [-32, 31] kept as
# u = c + 32; weights in groups of 16, u[i] the i-th of a group.
#   low plane  [N, K/2]: group byte j < 8 = (u[j] & 15) | (u[j + 8] & 15) << 4
#   high plane [N, K/4]: group byte j < 4 = sum over r < 4 of (u[j + 4 r] >> 4) << 2 r

KQ6_SHAPES = [("o", 4096, 4096), ("down", 12288, 4096)]
SEED_KQ6 = 8001


def kq6_pack(codes: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """codes int8 [N, K] in [-32, 31] -> (low plane uint8 [N, K/2], high plane uint8 [N, K/4])."""
    N, K = codes.shape
    assert K % 256 == 0 and codes.min() >= -32 and codes.max() <= 31
    u = (codes.astype(np.int16) + 32).astype(np.uint8).reshape(N, K // 16, 16)
    lo = u & 15
    ql = lo[:, :, :8] | (lo[:, :, 8:] << 4)
    hi = u >> 4
    qh = hi[:, :, 0:4] | (hi[:, :, 4:8] << 2) | (hi[:, :, 8:12] << 4) | (hi[:, :, 12:16] << 6)
    return ql.reshape(N, K // 2).astype(np.uint8), qh.reshape(N, K // 4).astype(np.uint8)


def kq6_weights(g: np.random.Generator, N: int, K: int):
    """-> (codes int8 [N, K], sub-scales int8 [N, K/16], superblock scales fp16 bits [N, K/256])."""
    codes = g.integers(-32, 32, (N, K), dtype=np.int8)
    sc = g.integers(-127, 128, (N, K // 16), dtype=np.int8)
    d = np.exp(g.uniform(np.log(1e-6), np.log(1e-4), (N, K // 256))).astype(np.float32)
    return codes, sc, d.astype(np.float16).view(np.uint16)


@dataclass
class KQ6Layer:
    name: str
    K: int
    N: int
    codes: np.ndarray    # int8 [N, K]
    ql: np.ndarray       # uint8 [N, K/2]
    qh: np.ndarray       # uint8 [N, K/4]
    sc: np.ndarray       # int8 [N, K/16]
    d: np.ndarray        # fp16 bits [N, K/256]
    x: np.ndarray        # bf16 bits [T, K]


def kq6_layer(i: int, tokens: int = 16) -> KQ6Layer:
    """Qwen3-8B o (4096 -> 4096) or down (12288 -> 4096) projection as kq6 weights."""
    name, K, N = KQ6_SHAPES[i]
    g = rng(SEED_KQ6 + i)
    codes, sc, d = kq6_weights(g, N, K)
    ql, qh = kq6_pack(codes)
    x = normal_bf16(g, tokens, K)
    return KQ6Layer(name, K, N, codes, ql, qh, sc, d, x)


# -- kq4: 4-bit codes with a sub-scale and a minimum per 32 weights --------------------
#
# Layout (this library's own): codes q in [0, 15] in the kq6 low plane (group
# byte j < 8 of each 16 weights = q[j] | q[j + 8] << 4); scm [N, K/32, 2] uint8 = (sub-scale, minimum) per 32
# weights, both in [0, 63]; dm [N, K/256, 2] fp16 = (d, dmin) per superblock.

def kq4_pack(codes: np.ndarray) -> np.ndarray:
    """codes uint8 [N, K] in [0, 15] -> low plane uint8 [N, K/2]."""
    assert codes.min() >= 0 and codes.max() <= 15
    N, K = codes.shape
    c = codes.astype(np.uint8).reshape(N, K // 16, 16)
    return (c[:, :, :8] | (c[:, :, 8:] << 4)).reshape(N, K // 2).astype(np.uint8)


def kq4_weights(g: np.random.Generator, N: int, K: int):
    """-> (codes uint8 [N, K], scm uint8 [N, K/32, 2], dm fp16 bits [N, K/256, 2])."""
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    scm = g.integers(0, 64, (N, K // 32, 2), dtype=np.uint8)
    d = np.exp(g.uniform(np.log(1e-5), np.log(1e-3), (N, K // 256)))
    dmin = np.exp(g.uniform(np.log(1e-4), np.log(1e-2), (N, K // 256)))
    dm = np.stack([d, dmin], axis=-1).astype(np.float32).astype(np.float16).view(np.uint16)
    return codes, scm, dm


@dataclass
class KQ4Layer:
    name: str
    K: int
    N: int
    codes: np.ndarray    # uint8 [N, K]
    ql: np.ndarray       # uint8 [N, K/2]
    scm: np.ndarray      # uint8 [N, K/32, 2]
    dm: np.ndarray       # fp16 bits [N, K/256, 2]
    x: np.ndarray        # bf16 bits [T, K]


SEED_KQ4 = 9001


def kq4_layer(i: int, tokens: int = 16) -> KQ4Layer:
    """Qwen3-8B o (4096 -> 4096) or down (12288 -> 4096) projection as kq4 weights."""
    name, K, N = KQ6_SHAPES[i]
    g = rng(SEED_KQ4 + i)
    codes, scm, dm = kq4_weights(g, N, K)
    x = normal_bf16(g, tokens, K)
    return KQ4Layer(name, K, N, codes, kq4_pack(codes), scm, dm, x)
