"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and lays them out; it holds none of the
softmax arithmetic.  Every array is reproducible from its seed alone.

Generation recipe (all configurations): the array is cut into blocks of whole
rows holding at most ``BLOCK_ELEMS`` elements; block ``b`` draws from
``numpy.random.Generator(PCG64(seed).jumped(b))``, so blocks can be generated
in any order or in parallel and a row range can be regenerated without the
rest.  Within a block the draws come in the order each recipe lists.

The five workloads (shapes and value distributions of the benchmark
configurations; seeds 1001..1005):

1. ``[64, 1024]`` fp32, N(0, 1).
2. ``[4096, 32000]`` fp32 LM-logit rows: 2*N(0, 1); then each entry
   independently becomes +-80 with probability 1e-3 (sign by a fair coin);
   then each entry independently becomes -inf with probability 1e-4.  No row
   is entirely -inf (checked).
3. ``[524288, 2048]`` bf16 attention-score rows (8 batch x 32 heads x 2048
   queries): N(0, 1) * (1/sqrt(128)) in fp32, rounded to bf16 to nearest-even;
   returned as uint16 bit patterns.
4. ``[8388608, 128]`` fp32 short rows, U(-10, 10).
5. ``[256, 128256]`` fp32 top-K rows, 3*N(0, 1); then 13 rows (5% of 256,
   chosen without replacement) get their maximum copied to 1-3 further
   distinct positions, one of them before the original maximum when it is
   not at position 0.  These draws use ``PCG64(seed).jumped(1 << 20)``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK_ELEMS = 1 << 24
SEED_BASE = 1000

SHAPES = {
    1: (64, 1024),
    2: (4096, 32000),
    3: (524288, 2048),
    4: (8388608, 128),
    5: (256, 128256),
}
DTYPES = {1: "f32", 2: "f32", 3: "bf16", 4: "f32", 5: "f32"}
TOPK_K = 8
INV_SQRT_128 = np.float32(1.0 / math.sqrt(128.0))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed).jumped(block))


def rows_per_block(cols: int) -> int:
    return max(1, BLOCK_ELEMS // max(1, cols))


def _blocked(rows, cols, seed, fill, out_dtype, row_start=0, row_stop=None):
    """Run ``fill(gen, nrows) -> array[nrows, cols]`` per block; keep rows [start, stop)."""
    if row_stop is None:
        row_stop = rows
    rpb = rows_per_block(cols)
    b0, b1 = row_start // rpb, -(-row_stop // rpb)
    out = np.empty((row_stop - row_start, cols), dtype=out_dtype)

    def work(b):
        r0 = b * rpb
        r1 = min(rows, r0 + rpb)
        blk = fill(_gen(seed, b), r1 - r0)
        lo, hi = max(r0, row_start), min(r1, row_stop)
        out[lo - row_start:hi - row_start] = blk[lo - r0:hi - r0]

    blocks = range(b0, b1)
    if len(blocks) <= 1:
        for b in blocks:
            work(b)
    else:
        with ThreadPoolExecutor(max_workers=_threads()) as pool:
            list(pool.map(work, blocks))
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 to bf16, nearest-even; uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# -- generic seeded rows (edge cases, small parity cases) ----------------------

def normal(rows, cols, seed, scale=1.0):
    s = np.float32(scale)
    return _blocked(rows, cols, seed,
                    lambda g, n: g.standard_normal((n, cols), dtype=np.float32) * s,
                    np.float32)


def uniform(rows, cols, seed, lo=-10.0, hi=10.0):
    return _blocked(rows, cols, seed,
                    lambda g, n: g.uniform(lo, hi, (n, cols)).astype(np.float32),
                    np.float32)


def grid_values(rows, cols, seed, step_log2=-10, bound=8.0):
    """Values on the grid k * 2**step_log2 with |x| < bound (shift tests)."""
    q = int(bound * 2 ** (-step_log2))

    def fill(g, n):
        k = g.integers(-q + 1, q, size=(n, cols))
        return np.ldexp(k.astype(np.float64), step_log2).astype(np.float32)

    return _blocked(rows, cols, seed, fill, np.float32)


# -- the five workloads ---------------------------------------------------------

def _fill_cfg2(g, n):
    cols = SHAPES[2][1]
    x = g.standard_normal((n, cols), dtype=np.float32) * np.float32(2.0)
    big = g.random((n, cols), dtype=np.float32) < np.float32(1e-3)
    sign = g.random((n, cols), dtype=np.float32) < np.float32(0.5)
    x[big & sign] = np.float32(80.0)
    x[big & ~sign] = np.float32(-80.0)
    neg = g.random((n, cols), dtype=np.float32) < np.float32(1e-4)
    x[neg] = -np.inf
    return x


def _fill_cfg3(g, n):
    cols = SHAPES[3][1]
    x = g.standard_normal((n, cols), dtype=np.float32) * INV_SQRT_128
    return f32_to_bf16_bits(x)


def _dup_maxima(x: np.ndarray, seed: int):
    rows, cols = x.shape
    g = _gen(seed, 1 << 20)
    n_dup = int(round(0.05 * rows))
    picked = np.sort(g.choice(rows, size=n_dup, replace=False))
    for r in picked:
        a = int(np.argmax(x[r]))
        copies = int(g.integers(1, 4))
        used = {a}
        positions = []
        if a > 0:
            p = int(g.integers(0, a))
            used.add(p)
            positions.append(p)
        while len(positions) < copies:
            p = int(g.integers(0, cols))
            if p not in used:
                used.add(p)
                positions.append(p)
        x[r, positions] = x[r, a]
    return picked


def config(n: int, row_start: int = 0, row_stop: int | None = None) -> np.ndarray:
    """Rows [row_start, row_stop) of workload ``n`` (fp32, or uint16 bf16 bits)."""
    rows, cols = SHAPES[n]
    seed = SEED_BASE + n
    row_stop = rows if row_stop is None else min(row_stop, rows)
    row_start = min(row_start, row_stop)
    if n == 1:
        fill, dt = (lambda g, k: g.standard_normal((k, cols), dtype=np.float32)), np.float32
    elif n == 2:
        fill, dt = _fill_cfg2, np.float32
    elif n == 3:
        fill, dt = _fill_cfg3, np.uint16
    elif n == 4:
        fill, dt = (lambda g, k: g.uniform(-10.0, 10.0, (k, cols)).astype(np.float32)), np.float32
    elif n == 5:
        if row_start != 0 or row_stop != rows:
            full = config(5)
            return np.ascontiguousarray(full[row_start:row_stop])
        fill, dt = (lambda g, k: g.standard_normal((k, cols), dtype=np.float32) * np.float32(3.0)), np.float32
    else:
        raise ValueError(f"unknown workload {n}")
    x = _blocked(rows, cols, seed, fill, dt, row_start, row_stop)
    if n == 5:
        _dup_maxima(x, seed)
    return x


def dup_rows_cfg5() -> np.ndarray:
    """Indices of the rows of workload 5 that carry duplicated maxima."""
    rows, cols = SHAPES[5]
    x = _blocked(rows, cols, SEED_BASE + 5,
                 lambda g, k: g.standard_normal((k, cols), dtype=np.float32) * np.float32(3.0),
                 np.float32)
    return _dup_maxima(x, SEED_BASE + 5)


# -- attention inputs ---------------------------------------------------------------
#
# The attention forward's workload takes workload 3's shape as an attention
# problem: 8 batch x 32 heads = 256 heads of 2048 queries and 2048 keys, head
# dimension 128 (the 1/sqrt(128) scale of workload 3), Q, K and V drawn
# N(0, 1) in fp32 and rounded to bf16 nearest-even, seeds 1006 (Q), 1007 (K),
# 1008 (V), laid out [heads, n, d].
ATTN_HEADS, ATTN_N, ATTN_D = 8 * 32, 2048, 128
ATTN_SEED = 1006


def attention_qkv(heads: int, nq: int, nk: int, d: int, seed: int):
    """Seeded bf16 Q [heads, nq, d], K and V [heads, nk, d] (uint16 bit patterns),
    each N(0, 1) rounded to nearest-even, from seeds seed, seed + 1, seed + 2."""
    def draw(n, s):
        x = _blocked(heads * n, d, s, lambda g, m: g.standard_normal((m, d), dtype=np.float32), np.float32)
        return f32_to_bf16_bits(x).reshape(heads, n, d)
    return draw(nq, seed), draw(nk, seed + 1), draw(nk, seed + 2)


def attention_workload():
    """The attention workload: (q, k, v) of 256 heads x 2048 x 128."""
    return attention_qkv(ATTN_HEADS, ATTN_N, ATTN_N, ATTN_D, ATTN_SEED)


def two_shard_row() -> np.ndarray:
    """The worked example's row: shard A = [1, 2], shard B = [3]."""
    return np.array([[1.0, 2.0, 3.0]], dtype=np.float32)


def mock_row() -> np.ndarray:
    """The lesson's unit-test vector with large and very negative entries."""
    return np.array([[1.0, 2.0, 10.0, 85.0, 87.0, -50.0]], dtype=np.float32)
