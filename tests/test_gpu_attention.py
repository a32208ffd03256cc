"""GPU parity of the batch-invariant decode attention (tolerance 0 ulp):
the oracle on every row at small sizes (ragged contexts, chunk edges, every
query-heads-per-kv-head ratio), each row of a verify batch against the same
token decoded alone, the cache's allocation and strides, and Qwen3-8B shapes
at long context on sampled heads.  Cache slots past the written cells hold
NaN, so a read past a query's position would show in its output."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import assert_bits_equal, dev, host_bits, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def iqd():
    import invariant_quantized_decode_token_amd as m

    m.load()
    return m


def run(iqd, case, q=None, pos0=None, k=None, v=None):
    q = case.q if q is None else q
    pos0 = case.pos0 if pos0 is None else pos0
    kd = dev(case.k) if k is None else k
    vd = dev(case.v) if v is None else v
    return host_bits(iqd.attn_decode(dev(q), kd, vd, pos0, float(case.scale)))


@pytest.mark.parametrize("cells", [1, 5, 255, 256, 257, 300, 511, 512, 513, 1000, 2049])
def test_oracle_parity_ragged_contexts(iqd, cells):
    for b in (1, 3, 8, 16):
        if b > cells:
            continue
        case = W.attn_case(W.SEED_ATTN + cells * 17 + b, b, cells, Hq=8, Hkv=2, capacity=cells + 37)
        got = run(iqd, case)
        want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale)
        assert_bits_equal(got, want, f"cells={cells} b={b}")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_oracle_parity_head_ratios(iqd, G):
    Hkv = 2
    for cells, b in ((200, 5), (777, 5), (1290, 9)):
        case = W.attn_case(W.SEED_ATTN + 100 * G + cells, b, cells, Hq=G * Hkv, Hkv=Hkv, capacity=cells + 8)
        got = run(iqd, case)
        want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale)
        assert_bits_equal(got, want, f"G={G} cells={cells} b={b}")


@pytest.mark.parametrize("pos0", [250, 504, 1020])
def test_batch_across_a_chunk_edge(iqd, pos0):
    """Rows of one launch on both sides of a 256-cell edge: some finish in
    one chunk fewer than others (at pos0 = 250, some take the fast path and
    some the merge)."""
    b = 12
    case = W.attn_case(W.SEED_ATTN + pos0, b, pos0 + b, Hq=32, Hkv=8, capacity=pos0 + b + 300)
    got = run(iqd, case)
    want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale)
    assert_bits_equal(got, want, f"pos0={pos0}")


def test_every_batch_row_equals_the_token_alone(iqd):
    """A sequence of 48 queries at positions 1100..1147 replayed in verify
    batches of every size b = 1..16 (consecutive chunks of the sequence, the
    last one short): every row equals that token decoded alone."""
    n, start = 48, 1100
    case = W.attn_case(W.SEED_ATTN + 7, n, start + n, capacity=start + n + 64)
    kd, vd = dev(case.k), dev(case.v)
    alone = np.stack([run(iqd, case, q=case.q[t:t + 1], pos0=start + t, k=kd, v=vd)[0] for t in range(n)])
    rows = [0, 5, 17, 31]
    want = np.zeros_like(alone)
    want[:, rows] = oracle.attn_decode(case.q, case.k, case.v, start, case.scale, heads=(0, 32))[:, rows]
    assert_bits_equal(alone[:, rows], want[:, rows], "b=1 vs oracle")
    for b in range(2, 17):
        for t0 in range(0, n, b):
            t1 = min(n, t0 + b)
            got = run(iqd, case, q=case.q[t0:t1], pos0=start + t0, k=kd, v=vd)
            assert_bits_equal(got, alone[t0:t1], f"b={b} window at {t0}")


def test_cache_allocation_and_strides_do_not_matter(iqd):
    """The same cells held (a) in exact-size caches, (b) in a 4x larger
    allocation, (c) as strided K and V views of one packed [cells, 2, Hkv, D]
    buffer, (d) head-major [Hkv, cells, D] views: identical bits."""
    t = torch()
    b, cells, Hkv, D = 8, 1500, 8, 128
    case = W.attn_case(W.SEED_ATTN + 11, b, cells, capacity=cells)
    ref = run(iqd, case)
    big = W.attn_case(W.SEED_ATTN + 11, b, cells, capacity=4 * cells)
    assert np.array_equal(big.k[:cells], case.k[:cells])
    assert_bits_equal(run(iqd, big), ref, "4x allocation")
    packed = np.full((cells + 100, 2, Hkv, D), W.BF16_NAN, np.uint16)
    packed[:cells, 0] = case.k
    packed[:cells, 1] = case.v
    pd = dev(packed)
    assert_bits_equal(run(iqd, case, k=pd[:, 0], v=pd[:, 1]), ref, "packed K/V views")
    hm_k = dev(np.ascontiguousarray(case.k.transpose(1, 0, 2)))
    hm_v = dev(np.ascontiguousarray(case.v.transpose(1, 0, 2)))
    assert_bits_equal(run(iqd, case, k=hm_k.transpose(0, 1), v=hm_v.transpose(0, 1)), ref, "head-major views")
    assert hm_k.transpose(0, 1).stride() == (D, cells * D, 1)
    del t


@pytest.mark.parametrize("cells,b", [(4100, 8), (8300, 3), (16500, 2), (2049, 8), (5600, 3), (9000, 2)])
def test_row_groups_of_eight(iqd, cells, b):
    """Qwen3-8B heads at contexts long enough for workgroups of 8 rows that
    still number two per CU on a 256-CU chip: 32 rows as four full groups
    (4100 cells), 12 rows as a full group and a ragged one of 4 (8300), 8 rows
    as one (16500); shorter contexts take groups of 4 rows.  Sampled heads
    against the oracle; every row equals its token decoded alone."""
    case = W.attn_case(W.SEED_ATTN + 3 * cells + b, b, cells)
    kd, vd = dev(case.k), dev(case.v)
    got = run(iqd, case, k=kd, v=vd)
    for h in (0, 5, 22, 31):
        want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale, heads=(h, h + 1))
        assert_bits_equal(got[:, h], want[:, h], f"cells={cells} b={b} head={h}")
    for t in range(b):
        alone = run(iqd, case, q=case.q[t:t + 1], pos0=case.pos0 + t, k=kd, v=vd)
        assert_bits_equal(alone[0], got[t], f"cells={cells} b={b} token {t} alone")


def test_merge_over_many_windows(iqd):
    """70001 cells: 274 chunks per row, merged in windows of chunks with a
    ragged last window; two tokens, every head against the oracle, and each
    row against its token decoded alone."""
    b, cells = 2, 70001
    case = W.attn_case(W.SEED_ATTN + cells, b, cells, Hq=8, Hkv=2)
    kd, vd = dev(case.k), dev(case.v)
    got = run(iqd, case, k=kd, v=vd)
    want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale)
    assert_bits_equal(got, want, "70001 cells")
    for t in range(b):
        alone = run(iqd, case, q=case.q[t:t + 1], pos0=case.pos0 + t, k=kd, v=vd)
        assert_bits_equal(alone[0], got[t], f"token {t} alone")


@pytest.mark.parametrize("cells", [16129, 16385, 32769, 33025])
def test_merge_window_edges(iqd, cells):
    """Rows whose chunk counts sit on the merge's 64-chunk window edges: a
    3-token batch at the end of the context puts its rows at 63 / 63 / 64,
    64 / 64 / 65, 128 / 128 / 129 and 129 / 129 / 130 chunks (one launch,
    rows of different chunk counts), every output bit against the oracle."""
    b = 3
    case = W.attn_case(W.SEED_ATTN + cells + 5, b, cells, Hq=4, Hkv=1, capacity=cells + 3)
    got = run(iqd, case)
    want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale)
    assert_bits_equal(got, want, f"cells={cells}")


@pytest.mark.parametrize("cells", [4096, 32768])
def test_qwen3_8b_long_context_sampled_heads(iqd, cells):
    """Qwen3-8B attention (32 query heads, 8 kv heads, D = 128), b = 8 verify
    batch at the end of the context: heads 0, 13, 31 against the oracle, and
    every row equal to its token decoded alone."""
    b = 8
    case = W.attn_case(W.SEED_ATTN + cells, b, cells)
    kd, vd = dev(case.k), dev(case.v)
    got = run(iqd, case, k=kd, v=vd)
    for h in (0, 13, 31):
        want = oracle.attn_decode(case.q, case.k, case.v, case.pos0, case.scale, heads=(h, h + 1))
        assert_bits_equal(got[:, h], want[:, h], f"cells={cells} head={h}")
    for t in range(b):
        alone = run(iqd, case, q=case.q[t:t + 1], pos0=case.pos0 + t, k=kd, v=vd)
        assert_bits_equal(alone[0], got[t], f"cells={cells} token {t} alone")
