"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each pin takes an ``oracle.Oracle`` handle and raises ``AssertionError`` when
the oracle disagrees with: a value printed on the pages (fixtures under
``tests/golden/``), a closed form, a library routine (scipy, numpy, torch), an
algebraic law of the operator, or a brute-force enumeration.  The same pins run
against deliberately broken copies of ``oracle.c`` in ``test_oracle_mutants.py``
to show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


# -- values printed on the pages -------------------------------------------------

def pin_two_shard_worked_example(o):
    """Lesson 7's two-shard example: printed to 6 decimals, closed forms exactly."""
    g = _golden("two_shard_example.json")
    p = g["printed"]
    tol = 10.0 ** -g["printed_decimals"]
    ma, da = o.online_state(g["shard_a"])
    mb, db = o.online_state(g["shard_b"])
    mab, dab = o.combine((ma, da), (mb, db))
    assert ma == p["m_a"] and mb == p["m_b"] and mab == p["m_ab"]
    assert abs(da - p["d_a"]) <= tol and abs(db - p["d_b"]) <= tol and abs(dab - p["d_ab"]) <= tol
    assert _rel(da, 1.0 + math.exp(-1.0)) <= 1e-15
    assert _rel(dab, 1.0 + math.exp(-1.0) + math.exp(-2.0)) <= 1e-15
    # the page's global 3-pass check: d = e^-2 + e^-1 + 1 (each term printed)
    m3, d3 = o.stats(workloads.two_shard_row())
    assert m3[0] == 3.0
    assert abs(d3[0] - sum(g["printed"]["global_d_terms"])) <= 3 * tol
    assert _rel(d3[0], dab) <= 1e-15
    y = o.softmax(workloads.two_shard_row())[0]
    for k in range(3):
        assert _rel(y[k], math.exp(k - 2.0) / (1.0 + math.exp(-1.0) + math.exp(-2.0))) <= 1e-15


def pin_lesson_mock_vector(o):
    """Lesson 7's NumPy unit-test vector: 85/87 reduce to the logistic function."""
    g = _golden("lesson_mock_vector.json")
    x = np.array([g["input"]], dtype=np.float32)
    y = o.softmax(x)[0]
    sig2 = 1.0 / (1.0 + math.exp(-2.0))
    assert _rel(y[4], sig2) <= 1e-15
    assert _rel(y[3], 1.0 - sig2) <= 1e-14
    assert abs(y.sum() - 1.0) <= g["sum_atol"]
    assert np.all(y[[0, 1, 2, 5]] < 1e-33)
    # the chunked online fold of the page equals the plain 3-pass statistics
    c = g["chunk_size"]
    state = (-math.inf, 0.0)
    for s in range(0, x.shape[1], c):
        state = o.combine(state, o.online_state(x[0, s:s + c]))
    m, d = o.stats(x)
    assert state[0] == m[0] and _rel(state[1], d[0]) <= 1e-15


# -- the induction base case, the bound and the identity -------------------------

def pin_base_case(o):
    """d_1 = 1 for any single finite element (induction base case)."""
    rng = np.random.Generator(np.random.PCG64(7))
    for v in list(rng.standard_normal(32) * 50) + [0.0, -0.0, 3.0e38, -3.0e38, 1e-40]:
        m, d = o.online_state([float(np.float32(v))])
        assert m == float(np.float32(v)) and d == 1.0


def pin_bound(o):
    """1 <= d <= N for every row (the recurrence's invariant), in double."""
    x = workloads.normal(64, 777, seed=11, scale=4.0)
    x[3, ::5] = -np.inf
    m, d = o.stats(x)
    assert np.all(d >= 1.0) and np.all(d <= x.shape[1])
    for r in range(0, 64, 9):
        mo, do = o.online_state(x[r])
        assert 1.0 <= do <= x.shape[1]


def pin_identity(o):
    """(-inf, 0) is a two-sided identity of the operator, exactly."""
    ident = (-math.inf, 0.0)
    for s in [(2.0, 1.3678794411714423), (-7.5, 3.0), (80.0, 16.0), ident]:
        assert o.combine(s, ident) == s
        assert o.combine(ident, s) == s
    assert o.online_state([]) == ident
    assert o.online_state([-math.inf, -math.inf]) == ident
    m, d = o.stats(np.full((1, 5), -np.inf, dtype=np.float32))
    assert m[0] == -math.inf and d[0] == 0.0


# -- algebra of the operator --------------------------------------------------------

def _trees(states):
    """Every binary-tree reduction of ``states`` in the given order (Catalan many)."""
    if len(states) == 1:
        yield states[0]
        return
    for k in range(1, len(states)):
        for left in _trees(states[:k]):
            for right in _trees(states[k:]):
                yield ("node", left, right)


def _eval(o, t):
    if t[0] != "node":
        return t
    return o.combine(_eval(o, t[1]), _eval(o, t[2]))


def pin_operator_algebra(o):
    """Associativity and commutativity: every split and tree gives the plain (m, d)."""
    rng = np.random.Generator(np.random.PCG64(12))
    x = workloads.normal(24, 300, seed=13, scale=3.0)
    x[5, 17] = -np.inf
    x[6, :] = -np.inf
    x[6, 123] = 1.5
    m_ref, d_ref = o.stats(x)
    for r in range(x.shape[0]):
        cuts = np.sort(rng.choice(np.arange(0, 301), size=5))  # shards may be empty
        bounds = [0, *cuts.tolist(), 300]
        shards = [o.online_state(x[r, a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        left = shards[0]
        for s in shards[1:]:
            left = o.combine(left, s)
        right = shards[-1]
        for s in reversed(shards[:-1]):
            right = o.combine(s, right)
        perm = [shards[i] for i in rng.permutation(len(shards))]
        mixed = perm[0]
        for s in perm[1:]:
            mixed = o.combine(s, mixed) if rng.random() < 0.5 else o.combine(mixed, s)
        for st in (left, right, mixed):
            assert st[0] == m_ref[r]
            assert _rel(st[1], d_ref[r]) <= 1e-12
        a, b = shards[0], shards[1]
        assert o.combine(a, b) == o.combine(b, a)
    # brute force: every binary tree over 7 single-element states
    v = workloads.normal(1, 7, seed=14, scale=5.0)[0]
    leaves = [o.online_state([float(t)]) for t in v]
    m_ref, d_ref = o.stats(v[None, :])
    for t in _trees(leaves):
        m, d = _eval(o, t)
        assert m == m_ref[0] and _rel(d, d_ref[0]) <= 1e-14


def pin_recurrence_equals_definition(o):
    """The online recurrence reaches the 3-pass (m, d) (the induction proof)."""
    for seed, scale in [(21, 1.0), (22, 10.0), (23, 0.01)]:
        x = workloads.normal(8, 1000, seed=seed, scale=scale)
        m, d = o.stats(x)
        for r in range(8):
            mo, do = o.online_state(x[r])
            assert mo == m[r] and _rel(do, d[r]) <= 1e-12
    # a late maximum forces many rescalings
    ramp = np.arange(0, 500, dtype=np.float32)[None, :] * np.float32(0.05)
    m, d = o.stats(ramp)
    mo, do = o.online_state(ramp[0])
    assert mo == m[0] and _rel(do, d[0]) <= 1e-12


# -- library routines and textbook special cases ----------------------------------

def pin_scipy_softmax(o):
    """Equal to scipy.special.softmax / logsumexp in float64."""
    from scipy.special import logsumexp, softmax
    x = workloads.normal(32, 517, seed=31, scale=3.0)
    x[0, :7] = 80.0
    x[1, 3] = -np.inf
    y = o.softmax(x)
    ref = softmax(x.astype(np.float64), axis=1)
    assert np.max(np.abs(y - ref)) <= 1e-15
    pos = ref > 0
    assert np.array_equal(pos, y > 0)
    assert np.max(np.abs(y - ref)[pos] / ref[pos]) <= 1e-12
    m, d = o.stats(x)
    assert np.max(np.abs(m + np.log(d) - logsumexp(x.astype(np.float64), axis=1))) <= 1e-12


def pin_rows_sum_to_one(o):
    """Each row's outputs sum to 1 (in double, to 1e-12)."""
    for n in (1, 4, 2, 5):
        x = workloads.config(n, 0, 16) if n != 5 else workloads.config(5, 0, 4)
        y = o.softmax(x)
        assert np.all(np.abs(y.sum(axis=1) - 1.0) <= 1e-12)
    b = workloads.config(3, 0, 16)
    assert np.all(np.abs(o.softmax(b).sum(axis=1) - 1.0) <= 1e-12)


def pin_special_cases(o):
    """cols=1, two elements, equal rows, huge magnitudes, -inf/+inf/NaN entries."""
    assert o.softmax(np.array([[5.0], [-3e38]], dtype=np.float32)).tolist() == [[1.0], [1.0]]
    for a, b in [(0.5, -1.25), (10.0, 10.0), (-80.0, 80.0)]:
        y = o.softmax(np.array([[a, b]], dtype=np.float32))[0]
        assert _rel(y[0], 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
    for n in (1, 2, 64, 4096):
        y = o.softmax(np.full((2, n), 0.375, dtype=np.float32))
        assert np.all(y == 1.0 / n)
    y = o.softmax(np.array([[0.0, -1000.0], [1000.0, 1000.0], [-1000.0, -1000.0]], dtype=np.float32))
    assert y.tolist() == [[1.0, 0.0], [0.5, 0.5], [0.5, 0.5]]
    x = np.array([[1.0, -np.inf, 2.0, -np.inf]], dtype=np.float32)
    y = o.softmax(x)[0]
    assert y[1] == 0.0 and y[3] == 0.0 and _rel(y[2], 1.0 / (1.0 + math.exp(-1.0))) <= 1e-15
    assert np.all(np.isnan(o.softmax(np.full((1, 3), -np.inf, dtype=np.float32))))
    assert np.all(np.isnan(o.softmax(np.array([[1.0, np.inf, 0.0]], dtype=np.float32))))
    assert np.all(np.isnan(o.softmax(np.array([[1.0, np.nan, 0.0]], dtype=np.float32))))


def pin_shift_invariance(o):
    """softmax(x + c) == softmax(x) when the shift is exact (grid values, c = 64)."""
    x = workloads.grid_values(16, 333, seed=41)
    xs = x + np.float32(64.0)
    assert np.array_equal((xs - np.float32(64.0)), x)  # the shift is exact in fp32
    assert np.array_equal(o.softmax(x), o.softmax(xs))


def pin_bf16_widening(o):
    """bf16 inputs widen exactly: same result as torch's bf16 -> fp32 conversion."""
    import torch
    b = workloads.config(3, 0, 8)
    f = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(o.softmax(b), o.softmax(f))
    mb, db = o.stats(b)
    mf, df = o.stats(f)
    assert np.array_equal(mb, mf) and np.array_equal(db, df)


def pin_topk_library(o):
    """Top-K = numpy's stable argsort of -x (ties to the lowest index); probs = scipy softmax."""
    from scipy.special import softmax
    p, i = o.topk(np.array([[3, 5, 5, 1, 5]], dtype=np.float32), 5)
    assert i.tolist() == [[1, 2, 4, 0, 3]]
    rng = np.random.Generator(np.random.PCG64(51))
    x = rng.integers(-6, 7, size=(20, 97)).astype(np.float32)  # many exact ties
    x[3, :] = 2.0
    x[4, 10] = -0.0
    x[4, 11] = 0.0
    for K in (1, 8, 13, 97):
        p, i = o.topk(x, K)
        ref = np.argsort(-x.astype(np.float64), axis=1, kind="stable")[:, :K]
        assert np.array_equal(i, ref)
        full = softmax(x.astype(np.float64), axis=1)
        assert np.max(np.abs(p - np.take_along_axis(full, ref, axis=1))) <= 1e-15
    p, i = o.topk(x, 1)
    assert np.array_equal(i[:, 0], np.argmax(x, axis=1))
    w = workloads.config(5, 0, 2)
    p, i = o.topk(w, 8)
    ref = np.argsort(-w.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(i, ref)
    # bf16 rows (many exact ties after rounding): the same order on the widened values
    b = workloads.f32_to_bf16_bits(rng.standard_normal((12, 301)).astype(np.float32) * np.float32(0.05))
    b[2, :] = workloads.f32_to_bf16_bits(np.full((1, 301), 1.5, dtype=np.float32))[0]
    wide = workloads.bf16_bits_to_f32(b).astype(np.float64)
    for K in (1, 8, 32, 301):
        p, i = o.topk(b, K)
        ref = np.argsort(-wide, axis=1, kind="stable")[:, :K]
        assert np.array_equal(i, ref)
        assert np.max(np.abs(p - np.take_along_axis(softmax(wide, axis=1), ref, axis=1))) <= 1e-15


def pin_logsumexp(o):
    """logsumexp = scipy.special.logsumexp; closed forms; special rows; exp(x - L) = softmax."""
    from scipy.special import logsumexp, softmax
    x = workloads.normal(24, 389, seed=61, scale=4.0)
    x[0, :5] = 80.0
    x[1, 7] = -np.inf
    L = o.logsumexp(x)
    ref = logsumexp(x.astype(np.float64), axis=1)
    assert np.max(np.abs(L - ref)) <= 1e-13
    # L near 80 carries ~1e-14 of rounding, which exp(x - L) passes on
    assert np.max(np.abs(np.exp(x.astype(np.float64) - L[:, None]) - softmax(x.astype(np.float64), axis=1))) <= 1e-13
    b = workloads.config(3, 0, 8)
    f = b.view(np.int16).astype(np.int32) << 16
    fb = f.astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.max(np.abs(o.logsumexp(b) - logsumexp(fb, axis=1))) <= 1e-13
    # a + ln N for N equal entries; ln(e + e^2 + e^3); one element; two elements
    for a, n in ((0.375, 1), (-7.5, 2), (3.0, 1000), (80.0, 4096)):
        assert _rel(o.logsumexp(np.full((1, n), a, dtype=np.float32))[0], a + math.log(n)) <= 1e-15
    assert _rel(o.logsumexp(np.array([[1.0, 2.0, 3.0]], dtype=np.float32))[0],
                math.log(math.e + math.e ** 2 + math.e ** 3)) <= 1e-15
    assert o.logsumexp(np.array([[-3e38]], dtype=np.float32))[0] == np.float64(np.float32(-3e38))
    assert _rel(o.logsumexp(np.array([[0.5, -1.25]], dtype=np.float32))[0],
                0.5 + math.log1p(math.exp(-1.75))) <= 1e-15
    # -inf entries add nothing; all -inf gives -inf; empty rows give -inf
    assert o.logsumexp(np.array([[2.0, -np.inf, 1.0]], dtype=np.float32))[0] == \
        o.logsumexp(np.array([[2.0, 1.0]], dtype=np.float32))[0]
    assert o.logsumexp(np.full((1, 3), -np.inf, dtype=np.float32))[0] == -np.inf
    assert o.logsumexp(np.zeros((2, 0), dtype=np.float32)).tolist() == [-np.inf, -np.inf]
    assert np.isnan(o.logsumexp(np.array([[1.0, np.nan]], dtype=np.float32))[0])
    assert np.isnan(o.logsumexp(np.array([[1.0, np.inf]], dtype=np.float32))[0])
    # NaN next to nothing but -inf is still NaN (not the empty row's -inf)
    z = np.array([[-np.inf, np.nan, -np.inf], [np.nan, np.nan, np.nan]], dtype=np.float32)
    assert np.all(np.isnan(o.logsumexp(z)))
    m, d = o.stats(z)
    assert np.all(m == -np.inf) and np.all(np.isnan(d))
    assert np.all(np.isnan(o.softmax(z)))


def pin_naive_softmax(o):
    """The unshifted softmax of section 2: closed forms, scipy where e^x stays
    finite, and the overflow / underflow the page warns of, in double."""
    from scipy.special import softmax
    e = math.e
    y = o.naive_softmax(np.array([[1.0, 2.0, 3.0]], dtype=np.float32))[0]
    den = e + e * e + e ** 3
    for k in range(3):
        assert _rel(y[k], math.exp(k + 1.0) / den) <= 1e-15
    assert o.naive_softmax(np.array([[7.5]], dtype=np.float32)).tolist() == [[1.0]]
    a, b = 0.75, -2.5  # two entries: the logistic function of the difference
    y2 = o.naive_softmax(np.array([[a, b]], dtype=np.float32))[0]
    assert _rel(y2[0], 1.0 / (1.0 + math.exp(b - a))) <= 1e-15
    assert _rel(y2[1], 1.0 / (1.0 + math.exp(a - b))) <= 1e-15
    x = workloads.normal(16, 333, seed=71, scale=4.0)
    assert np.allclose(o.naive_softmax(x), softmax(x.astype(np.float64), axis=1), rtol=1e-13, atol=0)
    xb = workloads.f32_to_bf16_bits(workloads.normal(4, 99, seed=72, scale=2.0))
    wide = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    assert np.allclose(o.naive_softmax(xb), softmax(wide, axis=1), rtol=1e-13, atol=0)
    # -inf entries add e^{-inf} = 0
    xi = np.array([[1.0, -np.inf, 2.0, -np.inf]], dtype=np.float32)
    yi = o.naive_softmax(xi)[0]
    assert yi[1] == 0.0 and yi[3] == 0.0 and _rel(yi[2], 1.0 / (1.0 + math.exp(-1.0))) <= 1e-15
    # overflow: e^1000 is +inf in double, so the maximum's entry is inf/inf
    yo = o.naive_softmax(np.array([[1000.0, 0.0]], dtype=np.float32))[0]
    assert math.isnan(yo[0]) and yo[1] == 0.0
    # underflow: e^{-1000} is 0, so the whole row is 0/0
    assert np.all(np.isnan(o.naive_softmax(np.array([[-1000.0, -1000.0]], dtype=np.float32))))


def pin_topk_select(o):
    """Selection = numpy's stable argsort of -x (ties to the lowest index),
    values = the entries themselves; also on bf16 rows and K = cols."""
    v, i = o.topk_select(np.array([[3, 5, 5, 1, 5]], dtype=np.float32), 5)
    assert i.tolist() == [[1, 2, 4, 0, 3]] and v.tolist() == [[5.0, 5.0, 5.0, 3.0, 1.0]]
    rng = np.random.Generator(np.random.PCG64(73))
    x = rng.integers(-4, 5, size=(32, 301)).astype(np.float32)   # heavy ties
    x[::4] = workloads.normal(8, 301, seed=74, scale=3.0)
    x[1, :5] = [-0.0, 0.0, -0.0, 0.0, -0.0]                       # -0.0 ties +0.0
    x[2, 100:] = -np.inf
    for K in (1, 7, 32, 301):
        v, i = o.topk_select(x, K)
        ref = np.argsort(-x.astype(np.float64), axis=1, kind="stable")[:, :K]
        assert np.array_equal(i, ref), K
        assert np.array_equal(v, np.take_along_axis(x, ref, axis=1).astype(np.float64)), K
    xb = workloads.f32_to_bf16_bits(workloads.normal(6, 200, seed=75, scale=2.0))
    wide = workloads.bf16_bits_to_f32(xb).astype(np.float64)
    v, i = o.topk_select(xb, 9)
    ref = np.argsort(-wide, axis=1, kind="stable")[:, :9]
    assert np.array_equal(i, ref) and np.array_equal(v, np.take_along_axis(wide, ref, axis=1))


def _attn_inputs(heads, nq, nk, d, seed, scale_q=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = workloads.f32_to_bf16_bits((rng.standard_normal((heads, nq, d)) * scale_q).astype(np.float32))
    k = workloads.f32_to_bf16_bits(rng.standard_normal((heads, nk, d)).astype(np.float32))
    v = workloads.f32_to_bf16_bits(rng.standard_normal((heads, nk, d)).astype(np.float32))
    return q, k, v


def _wide(b):
    return workloads.bf16_bits_to_f32(b).astype(np.float64)


def pin_attention_library(o):
    """O = softmax(scale Q K^T) V and L = logsumexp by scipy in float64 (the
    three stages of section 7.1 written with library routines), with and
    without the causal mask; a subset of query rows equals those rows."""
    from scipy.special import logsumexp, softmax
    q, k, v = _attn_inputs(3, 37, 53, 24, seed=81)
    scale = 1.0 / math.sqrt(24)
    O, L = o.attention(q, k, v, scale)
    X = np.einsum("hic,hjc->hij", _wide(q), _wide(k)) * scale
    assert np.allclose(O, softmax(X, axis=-1) @ _wide(v), rtol=0, atol=1e-12)
    assert np.allclose(L, logsumexp(X, axis=-1), rtol=1e-13, atol=0)
    qs, ks, vs = _attn_inputs(2, 40, 40, 16, seed=82)
    Oc, Lc = o.attention(qs, ks, vs, 0.3, causal=True)
    Xc = np.einsum("hic,hjc->hij", _wide(qs), _wide(ks)) * 0.3
    Xc = np.where(np.tril(np.ones((40, 40), dtype=bool)), Xc, -np.inf)  # key j hidden from query i when j > i
    assert np.allclose(Oc, softmax(Xc, axis=-1) @ _wide(vs), rtol=0, atol=1e-12)
    assert np.allclose(Lc, logsumexp(Xc, axis=-1), rtol=1e-13, atol=0)
    Os, Ls = o.attention(np.ascontiguousarray(qs[:, 11:29]), ks, vs, 0.3, causal=True, q_off=11)
    assert np.array_equal(Os, Oc[:, 11:29]) and np.array_equal(Ls, Lc[:, 11:29])


def pin_attention_closed_forms(o):
    """Equal keys: the mean of V; one key: V itself; V of ones: ones; two keys:
    the logistic mix; causal row 0: V[0]; a huge scale: the argmax key's V;
    the |V| weights equal O for V >= 0."""
    bits = workloads.f32_to_bf16_bits
    q, k, v = _attn_inputs(2, 9, 6, 8, seed=83)
    k_eq = np.ascontiguousarray(np.broadcast_to(k[:, :1], k.shape))
    O, L = o.attention(q, k_eq, v, 0.7)
    assert np.allclose(O, _wide(v).mean(axis=1, keepdims=True), rtol=0, atol=1e-15)
    s0 = 0.7 * np.einsum("hic,hc->hi", _wide(q), _wide(k)[:, 0])
    assert np.allclose(L, s0 + math.log(6), rtol=1e-15, atol=1e-14)
    O1, L1 = o.attention(q, k[:, :1].copy(), v[:, :1].copy(), 0.7)
    assert np.array_equal(O1, np.broadcast_to(_wide(v)[:, :1], O1.shape))
    assert np.allclose(L1, s0, rtol=1e-15, atol=0)
    ones = bits(np.ones(v.shape, dtype=np.float32))
    assert np.allclose(o.attention(q, k, ones, 0.7)[0], 1.0, rtol=0, atol=1e-15)
    O2 = o.attention(q, k[:, :2].copy(), v[:, :2].copy(), 0.7)[0]
    s = 0.7 * np.einsum("hic,hjc->hij", _wide(q), _wide(k)[:, :2])
    w0 = 1.0 / (1.0 + np.exp(s[..., 1] - s[..., 0]))
    ref = w0[..., None] * _wide(v)[:, None, 0] + (1 - w0)[..., None] * _wide(v)[:, None, 1]
    assert np.allclose(O2, ref, rtol=0, atol=1e-14)
    qc, kc, vc = _attn_inputs(1, 5, 5, 8, seed=84)
    Oc = o.attention(qc, kc, vc, 0.5, causal=True)[0]
    assert np.array_equal(Oc[0, 0], _wide(vc)[0, 0])
    # a very large scale: all weight on the largest logit (distinct logits)
    X = np.einsum("hic,hjc->hij", _wide(q), _wide(k))
    Oh = o.attention(q, k, v, 1.0e6)[0]
    assert np.allclose(Oh, np.take_along_axis(_wide(v), X.argmax(axis=-1)[..., None], axis=1), rtol=0, atol=1e-15)
    va = bits(np.abs(workloads.bf16_bits_to_f32(v)))
    Op, _, Oa = o.attention(q, k, va, 0.7, want_abs=True)
    assert np.allclose(Oa, Op, rtol=1e-15, atol=0)
    _, _, Oa2 = o.attention(q, k, v, 0.7, want_abs=True)
    assert np.array_equal(Oa2, Oa)


def pin_attention_tiled_recurrence(o):
    """The tiled (m, l, o~) recurrence with delayed rescaling reaches the
    definition for any tile size (the induction of section 3.2 carried to o),
    with and without the mask, also when a later tile raises the maximum."""
    q, k, v = _attn_inputs(2, 33, 70, 16, seed=85, scale_q=3.0)
    k[:, 66] = workloads.f32_to_bf16_bits(np.full((2, 16), 4.0, dtype=np.float32))  # a late, large logit
    for causal, nk in ((False, 70), (True, 33)):
        kk, vv = np.ascontiguousarray(k[:, :nk]), np.ascontiguousarray(v[:, :nk])
        O, L = o.attention(q, kk, vv, 0.25, causal=causal)
        for tile in (1, 3, 16, 64, nk):
            Ot, Lt = o.attention_tiled(q, kk, vv, 0.25, tile, causal=causal)
            assert np.allclose(Ot, O, rtol=0, atol=1e-13), (causal, tile)
            assert np.allclose(Lt, L, rtol=1e-14, atol=0), (causal, tile)


PINS = [
    pin_two_shard_worked_example,
    pin_lesson_mock_vector,
    pin_base_case,
    pin_bound,
    pin_identity,
    pin_operator_algebra,
    pin_recurrence_equals_definition,
    pin_scipy_softmax,
    pin_rows_sum_to_one,
    pin_special_cases,
    pin_shift_invariance,
    pin_bf16_widening,
    pin_topk_library,
    pin_logsumexp,
    pin_naive_softmax,
    pin_topk_select,
    pin_attention_library,
    pin_attention_closed_forms,
    pin_attention_tiled_recurrence,
]


def run_all(o):
    """Run every pin; return the names of those that failed."""
    failed = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            failed.append(pin.__name__)
    return failed

