"""Pins of the oracle's decode attention (fixed 256-cell chunks, fixed-order
merge) against what mathematics fixes: the exponential against the real
function, the output against softmax(q k^T) v formed in float64, two
closed forms (equal keys give the mean of the values; one dominant key
gives its value), the invariances the recipe promises (batch, position of
the window, cache allocation and strides), and the recipe's operation
order checked step by step in exact rational arithmetic on a small case.

Sources: "why speculative decoding changed my output", "the bug that waited
for position 384" (Fig. 5); "My speculative decoder got slower", "Fusion
that lost" and "Shipping the 6.4x as its own backend".
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W
from exact import bf16, bf16_bits_of, f32

SCALE = np.float32(1.0 / math.sqrt(128.0))


def bf16_vals(h):
    return (h.astype(np.uint32) << 16).view(np.float32)


def spacings(a, b):
    def key(h):
        h = h.astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)
    return np.abs(key(a) - key(b))


def test_exp_within_one_ulp_of_the_real_function():
    xs = np.concatenate([np.linspace(-86.5, 0.0, 60001, dtype=np.float32),
                         -np.logspace(-9, 1.93, 3000).astype(np.float32)])
    worst = 0.0
    for x in xs:
        e = float(oracle.attn_exp(x))
        t = math.exp(float(x))
        worst = max(worst, abs(e - t) / float(np.spacing(np.float32(t))))
    assert worst <= 1.0, worst
    assert float(oracle.attn_exp(0.0)) == 1.0 and float(oracle.attn_exp(-0.0)) == 1.0
    # below e^-86.6... (n < -125) the result is 0; just above, a normal number
    assert float(oracle.attn_exp(-87.0)) == 0.0 and float(oracle.attn_exp(-200.0)) == 0.0
    assert float(oracle.attn_exp(-86.5)) >= 2.0 ** -126


def random_case(seed, b, Hq, Hkv, D, cells):
    g = W.rng(seed)
    q = W.normal_bf16(g, b * Hq, D).reshape(b, Hq, D)
    k = W.normal_bf16(g, cells * Hkv, D).reshape(cells, Hkv, D)
    v = W.normal_bf16(g, cells * Hkv, D).reshape(cells, Hkv, D)
    return q, k, v


def truth_f64(q, k, v, pos0, scale):
    b, Hq, D = q.shape
    G = Hq // k.shape[1]
    qf, kf, vf = bf16_vals(q).astype(np.float64), bf16_vals(k).astype(np.float64), bf16_vals(v).astype(np.float64)
    out = np.empty((b, Hq, D))
    for t in range(b):
        p = pos0 + t
        for h in range(Hq):
            s = kf[:p + 1, h // G] @ qf[t, h] * float(scale)
            e = np.exp(s - s.max())
            out[t, h] = (e @ vf[:p + 1, h // G]) / e.sum()
    return out


def test_matches_float64_softmax_within_one_spacing():
    """Ragged context over three chunks (cells 0..700), GQA 4 to 1."""
    q, k, v = random_case(71, 3, 8, 2, 128, 704)
    pos0 = 698
    got = oracle.attn_decode(q, k, v, pos0, SCALE)
    want = truth_f64(q, k, v, pos0, SCALE)
    want_bits = W.f32_to_bf16_bits(want.astype(np.float32))  # two roundings: at most one spacing off
    d = spacings(got, want_bits)
    assert d.max() <= 1
    assert (d == 0).mean() > 0.995


@pytest.mark.parametrize("cells", [1, 200, 256, 257, 900])
def test_equal_keys_give_the_mean_of_the_values(cells):
    """Every score equal: e_j = 1, so l counts the cells and o sums the
    values; with small integer values every partial sum is exact and
    out = bf16(fl(sum / count)), whatever the chunk count."""
    g = W.rng(cells)
    D, Hkv = 128, 2
    krow = W.normal_bf16(g, 1, D)[0]
    k = np.broadcast_to(krow, (cells, Hkv, D)).copy()
    vals = g.integers(-8, 9, (cells, Hkv, D)).astype(np.float32)
    v = W.f32_to_bf16_bits(vals)
    q = W.normal_bf16(g, 4, D).reshape(1, 4, D)
    got = oracle.attn_decode(q, k, v, cells - 1, SCALE)
    for h in range(4):
        sums = vals[:, h // 2].astype(np.int64).sum(axis=0)
        for d in range(D):
            want = bf16_bits_of(float(bf16(f32(Fraction(int(sums[d]), cells)))))
            assert got[0, h, d] == want, (h, d, sums[d])


@pytest.mark.parametrize("star", [3, 255, 256, 600])
def test_one_dominant_key_gives_its_value(star):
    """One key scores about 181 above every other (q = 32 e_0, that key
    64 e_0): every other weight is E(< -87) = 0 exactly, so out = v_star."""
    g = W.rng(1000 + star)
    D, cells = 128, 700
    k = W.normal_bf16(g, cells, D).reshape(cells, 1, D)
    v = W.normal_bf16(g, cells, D).reshape(cells, 1, D)
    v[v == 0x8000] = 0x3F80  # no -0 values
    v[v == 0] = 0x3F80
    k[star, 0] = 0
    k[star, 0, 0] = W.f32_to_bf16_bits(np.float32([64.0]))[0]
    q = np.zeros((1, 1, D), np.uint16)
    q[0, 0, 0] = W.f32_to_bf16_bits(np.float32([32.0]))[0]
    got = oracle.attn_decode(q, k, v, cells - 1, SCALE)
    assert np.array_equal(got[0, 0], v[star, 0])


def test_results_do_not_depend_on_batch_window_or_cache_layout():
    """A query's row depends only on its own position: the same token at
    b = 1, inside a batch of 5 and of 9 (different pos0), and with the cache
    held as a strided view into a larger packed buffer, gives the same bits."""
    D, Hq, Hkv, cells = 128, 4, 2, 640
    q, k, v = random_case(9, 9, Hq, Hkv, D, cells)
    packed = np.zeros((cells + 64, 3, Hkv, D), np.uint16)  # [cells, (q?, k, v), heads, D]
    packed[:cells, 1] = k
    packed[:cells, 2] = v
    ks, vs = packed[:, 1], packed[:, 2]
    full = oracle.attn_decode(q, k, v, 500, SCALE)  # tokens at 500..508
    for t in range(9):
        alone = oracle.attn_decode(q[t:t + 1], k, v, 500 + t, SCALE)
        assert np.array_equal(alone[0], full[t])
        strided = oracle.attn_decode(q[t:t + 1], ks, vs, 500 + t, SCALE)
        assert np.array_equal(strided[0], full[t])
    five = oracle.attn_decode(q[4:9], k, v, 504, SCALE)
    assert np.array_equal(five, full[4:9])
    part = oracle.attn_decode(q, k, v, 500, SCALE, heads=(1, 3))
    assert np.array_equal(part[:, 1:3], full[:, 1:3])


# --- the recipe, re-derived in exact arithmetic --------------------------------

def _fma(a, b, c):
    return f32(a * b + c)


def _exp_exact(x):
    """The oracle's exponential with every binary32 step rounded exactly."""
    log2e = Fraction(float.fromhex("0x1.715476p+0"))
    hi = Fraction(float.fromhex("0x1.62e4p-1"))
    lo = Fraction(float.fromhex("0x1.7f7d1cp-20"))
    coef = [float.fromhex(h) for h in ("0x1.a01a02p-13", "0x1.6c16c2p-10", "0x1.111112p-7", "0x1.555556p-5",
                                       "0x1.555556p-3")] + [0.5, 1.0, 1.0]
    y = f32(x * log2e)
    n = math.floor(y)
    rem = y - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if n < -125:
        return Fraction(0)
    r = f32(f32(x - f32(n * hi)) - f32(n * lo))
    p = Fraction(coef[0])
    for c in coef[1:]:
        p = _fma(p, r, Fraction(c))
    return f32(p * Fraction(2) ** n)


def _recipe_exact(q, k, v, p, scale):
    """One row: q [D] and the cells 0..p of k, v ([cells, D]), as Fractions."""
    D = len(q)
    qs = [f32(Fraction(float(x)) * Fraction(float(scale))) for x in q]
    chunks = []
    for c0 in range(0, p + 1, 256):
        cells = range(c0, min(c0 + 256, p + 1))
        s = []
        for j in cells:
            part = []
            for l in range(D // 8):
                a = Fraction(0)
                for i in range(8 * l, 8 * l + 8):
                    a = _fma(qs[i], Fraction(float(k[j][i])), a)
                part.append(a)
            while len(part) > 1:
                part = [f32(part[2 * i] + part[2 * i + 1]) for i in range(len(part) // 2)]
            s.append(part[0])
        m = max(s)
        parts = []
        for a0 in range(c0, c0 + 256, 64):
            l_ = Fraction(0)
            o = [Fraction(0)] * D
            for j in range(a0, min(a0 + 64, p + 1)):
                e = _exp_exact(f32(s[j - c0] - m))
                l_ = f32(l_ + e)
                o = [_fma(e, Fraction(float(v[j][d])), o[d]) for d in range(D)]
            parts.append((l_, o))
        l_ = f32(f32(parts[0][0] + parts[1][0]) + f32(parts[2][0] + parts[3][0]))
        o = [f32(f32(parts[0][1][d] + parts[1][1][d]) + f32(parts[2][1][d] + parts[3][1][d])) for d in range(D)]
        chunks.append((m, l_, o))
    M = max(c[0] for c in chunks)
    L, O = None, None
    for i, (m, l_, o) in enumerate(chunks):
        w = _exp_exact(f32(m - M))
        if i == 0:
            L, O = f32(w * l_), [f32(w * x) for x in o]
        else:
            L, O = _fma(w, l_, L), [_fma(w, o[d], O[d]) for d in range(D)]
    return [bf16_bits_of(float(bf16(f32(x / L)))) for x in O]


def test_recipe_order_in_exact_arithmetic():
    """D = 16 (two slices), cells 0..299 (two chunks; the second ragged, with
    one part partly filled and two empty): every fl step of the recipe done
    exactly and rounded, against the C oracle bit for bit."""
    D, cells = 16, 300
    q, k, v = random_case(5, 1, 1, 1, D, cells)
    got = oracle.attn_decode(q, k, v, cells - 1, SCALE)
    qv = bf16_vals(q[0, 0])
    kv = bf16_vals(k[:, 0])
    vv = bf16_vals(v[:, 0])
    want = _recipe_exact(qv, kv, vv, cells - 1, SCALE)
    assert got[0, 0].tolist() == want


# --- witnesses of the fixed in-chunk order -----------------------------------------
# The pages fix chunking, partials and a merge but leave the float order inside
# a chunk open ("My speculative decoder got slower", "Shipping the 6.4x as its
# own backend": any one fixed rounding will do).  The recipe's order (8-dim
# score slices joined by an adjacent-pair tree; four 64-cell parts per chunk
# joined as (0 + 1) + (2 + 3)) is this library's choice.  Each witness below
# places the values 2^27, 1, -2^27, 1 (binary32 spacing 16 above 2^27 and 8
# below, so 2^27 + 1 and -2^27 + 1 both round back to +-2^27) so that the
# chosen order gives one result and each plausible alternative another; the
# expected outputs are worked out by hand in the docstrings.

BIG = W.f32_to_bf16_bits(np.float32([2.0 ** 27]))[0]
NBIG = W.f32_to_bf16_bits(np.float32([-(2.0 ** 27)]))[0]
ONE = W.f32_to_bf16_bits(np.float32([1.0]))[0]


def _part_case(cells_at):
    """One full chunk (256 cells, the query at position 255), q = 0 so every
    score is +0 and every weight E(0) = 1; dim 0 of the values holds the four
    witness values at the given cells, every other value is 0.  Then l = 256
    exactly and out[0] = bf16(o / 256) with o the chunk's sum of dim 0."""
    D = 128
    k = np.zeros((256, 1, D), np.uint16)
    v = np.zeros((256, 1, D), np.uint16)
    for cell, val in zip(cells_at, (BIG, ONE, NBIG, ONE)):
        v[cell, 0, 0] = val
    q = np.zeros((1, 1, D), np.uint16)
    return oracle.attn_decode(q, k, v, 255, SCALE)[0, 0]


def test_witness_chunk_parts_join_adjacent_pairs():
    """Values at cells 0, 64, 128, 192 (one per part): parts [2^27, 1, -2^27,
    1] joined (p0 + p1) + (p2 + p3) = 2^27 + -2^27 = 0.  A sequential sum over
    the chunk would give 1 (out 2^-8), pairing at stride two 2 (out 2^-7)."""
    out = _part_case((0, 64, 128, 192))
    assert out[0] == 0x0000
    assert np.all(out[1:] == 0)


def test_witness_parts_are_64_cells_not_128():
    """Cells 63, 64, 65, 66: part 0 ends at cell 63 (2^27), part 1 sums
    1, -2^27, 1 in order to -2^27, the join gives 0.  With 128-cell parts the
    four values would be one sequential run giving 1 (out 2^-8 = 0x3B80)."""
    assert _part_case((63, 64, 65, 66))[0] == 0x0000


def test_witness_parts_are_64_cells_not_32():
    """Cells 31, 32, 33, 34 lie in one 64-cell part, summed in order:
    ((2^27 + 1) - 2^27) + 1 = 1, out = bf16(1 / 256) = 2^-8.  With 32-cell
    parts they would split into 2^27 and -2^27 and give 0."""
    assert _part_case((31, 32, 33, 34))[0] == W.f32_to_bf16_bits(np.float32([2.0 ** -8]))[0]


def _score_case(kdims):
    """Two cells, the query (all ones, scale 1) at position 1.  Cell 0's key
    carries the witness values at the given dims, cell 1's key is zero (score
    0).  Values: cell 0 all 2, cell 1 all 4.  If cell 0 scores 0 both weights
    are 1 and out = (2 + 4) / 2 = 3 exactly."""
    D = 128
    k = np.zeros((2, 1, D), np.uint16)
    if kdims is not None:
        for d, val in zip(kdims, (BIG, ONE, NBIG, ONE)):
            k[0, 0, d] = val
    v = np.zeros((2, 1, D), np.uint16)
    v[0, 0, :] = W.f32_to_bf16_bits(np.float32([2.0]))[0]
    v[1, 0, :] = W.f32_to_bf16_bits(np.float32([4.0]))[0]
    q = np.full((1, 1, D), ONE, np.uint16)
    return q, k, v


def _score_out(kdims=None, plain_score=None):
    q, k, v = _score_case(kdims)
    if plain_score is not None:  # a key whose score is exactly plain_score: one nonzero dim
        k[0, 0, 0] = W.f32_to_bf16_bits(np.float32([plain_score]))[0]
    return oracle.attn_decode(q, k, v, 1, 1.0)[0, 0]


def test_witness_score_slices_join_adjacent_pairs():
    """Key dims 0, 8, 16, 24 (one per 8-dim slice): slice sums [2^27, 1, -2^27,
    1, 0, ...], the adjacent-pair tree gives 0, so out = 3.  A single chain
    over all 128 dims would score 1, stride pairing 2: both outputs differ."""
    out = _score_out((0, 8, 16, 24))
    three = W.f32_to_bf16_bits(np.float32([3.0]))[0]
    assert np.all(out == three)
    assert not np.array_equal(_score_out(plain_score=1.0), out)
    assert not np.array_equal(_score_out(plain_score=2.0), out)


def test_witness_score_slices_are_8_dims_not_16():
    """Key dims 7, 8, 9, 10: slice 0 ends at dim 7 (2^27), slice 1 chains
    1, -2^27, 1 to -2^27, the tree gives 0: out = 3.  16-dim slices would
    chain all four to 1."""
    three = W.f32_to_bf16_bits(np.float32([3.0]))[0]
    assert np.all(_score_out((7, 8, 9, 10)) == three)


def test_witness_score_slices_are_8_dims_not_4():
    """Key dims 3, 4, 5, 6 lie in slice 0, chained in order to 1: the row
    equals the row of a key that scores exactly 1.  4-dim slices would give
    score 0 and out = 3."""
    out = _score_out((3, 4, 5, 6))
    assert np.array_equal(out, _score_out(plain_score=1.0))
    assert not np.all(out == W.f32_to_bf16_bits(np.float32([3.0]))[0])
