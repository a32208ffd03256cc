"""Helpers for the GPU parity tests: numpy <-> torch device tensors and the
bitwise comparison used everywhere (tolerance 0 ulp)."""
from __future__ import annotations

import numpy as np


def torch():
    import torch as _t

    return _t


def dev(a: np.ndarray, dtype=None):
    """numpy -> cuda tensor; uint16 arrays become bf16 (dtype='bf16') or fp16 (dtype='fp16') bit patterns."""
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        x = t.from_numpy(a.view(np.int16))
        x = x.view(t.bfloat16 if dtype in (None, "bf16") else t.float16)
    else:
        x = t.from_numpy(a)
    return x.cuda()


def host_bits(x) -> np.ndarray:
    """bf16 / fp16 cuda tensor -> uint16 bit patterns on the host."""
    t = torch()
    return x.contiguous().view(t.int16).cpu().numpy().view(np.uint16)


def host(x) -> np.ndarray:
    return x.contiguous().cpu().numpy()


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} elements differ; first at {i}: "
                             f"got {got[i]!r} want {want[i]!r}")


def sample_rows(N: int, count: int, seed: int) -> np.ndarray:
    """Output rows to check against the oracle at full sizes: the first and
    last rows, rows around 64/256 boundaries and a seeded random sample."""
    g = np.random.default_rng(seed)
    fixed = [0, 1, N - 1, N - 2] + [r for r in (63, 64, 255, 256, 1023, 1024) if r < N]
    rnd = g.choice(N, size=min(count, N), replace=False).tolist()
    return np.array(sorted(set(fixed + rnd)), dtype=np.int64)
