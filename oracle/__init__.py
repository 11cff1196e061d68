"""CPU oracle for row-wise softmax with the online normalizer (double precision).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``online_normalizer_amd``) never does and fails loudly without its HIP library.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, no fast-math); this
module only loads it and marshals numpy arrays.  What each function computes,
with the passages it follows:

* ``softmax`` -- safe softmax in three passes (max, sum of e^{x-m}, divide):
  "OnlineSoftmax: Online normalizer calculation for softmax", section 2
  (safe softmax), and "CUDA算子优化(3)：Softmax", section "Softmax的cpu实现".
* ``stats`` -- the per-row state (m, d) by the same plain definition.
* ``logsumexp`` -- the per-row log(sum e^{x}) = m + log(d), the statistic that
  "6.2 FlashAttention V2 chi tiết" keeps for the backward pass (sections 6.1,
  7.1).
* ``online_state`` -- the element-by-element recurrence of section 3.1 of the
  paper summary, starting from the identity (-inf, 0) ("第 7 课：Online Softmax
  与可结合状态", section 3).
* ``combine`` -- the binary operator of section 3.3 of the paper summary.
* ``topk`` -- brute-force sort of the whole row under (value desc, index asc),
  probabilities e^{u-m}/d over the whole row (section 4 of the paper summary),
  for fp32 rows or bf16 rows (widened exactly).
* ``naive_softmax`` -- the unshifted softmax e^{x_i} / sum_j e^{x_j} in two
  passes, section 2 "Original softmax" of the paper summary, in double with
  no guard against overflow.
* ``topk_select`` -- the K largest entries of each row and their columns by
  the same sort, returned as the entries themselves: the TopK stage of the
  unfused pipelines in the access table of section 4 of the paper summary.
* ``attention`` -- O = softmax(scale Q K^T) V by the definition (section 7.1
  of the paper summary), optional causal mask, and the per-row logsumexp L =
  m + log(l) ("6.2 FlashAttention V2 chi tiết", sections 5, 6.1, 7.1), for
  bf16 Q, K, V of shape [heads, n, d].
* ``attention_tiled`` -- the same by the tiled (m, l, o~) recurrence with
  delayed rescaling (section 7.2.3 of the paper summary; "6.2 ...", sections
  3.2 and 6.1), tiles of b keys.

Rows are independent, so the wrappers may split a batch of rows over host
threads (each thread runs the same sequential C code on its own rows).
"""
from __future__ import annotations

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")


# Compiling the library lives in the ``oracle.build`` module
# (``from oracle.build import build``; ``python -m oracle.build``).
__all__ = ["Oracle", "load", "DEFAULT_LIB"]

_c_double_p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """Handle on one compiled copy of ``oracle.c``."""

    def __init__(self, path: str = DEFAULT_LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(
                f"oracle library {path} is missing; run __graft_entry__.build() "
                "or python -m oracle.build")
        self.path = path
        lib = ctypes.CDLL(path)
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        for name in ("oracle_softmax_f32", "oracle_softmax_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, vp]
            fn.restype = ctypes.c_int
        for name in ("oracle_stats_f32", "oracle_stats_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, vp, vp]
            fn.restype = ctypes.c_int
        for name in ("oracle_logsumexp_f32", "oracle_logsumexp_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, vp]
            fn.restype = ctypes.c_int
        lib.oracle_online_state.argtypes = [vp, i64, _c_double_p, _c_double_p]
        lib.oracle_online_state.restype = None
        lib.oracle_combine.argtypes = [ctypes.c_double] * 4 + [_c_double_p, _c_double_p]
        lib.oracle_combine.restype = None
        for name in ("oracle_topk_f32", "oracle_topk_bf16", "oracle_topk_select_f32", "oracle_topk_select_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
            fn.restype = ctypes.c_int
        lib.oracle_attention_bf16.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int, i64,
                                              vp, vp, vp]
        lib.oracle_attention_bf16.restype = ctypes.c_int
        lib.oracle_attention_tiled_bf16.argtypes = [vp, vp, vp, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                                    i64, i64, vp, vp]
        lib.oracle_attention_tiled_bf16.restype = ctypes.c_int
        for name in ("oracle_naive_softmax_f32", "oracle_naive_softmax_bf16"):
            fn = getattr(lib, name)
            fn.argtypes = [vp, i64, i64, vp]
            fn.restype = ctypes.c_int
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _split(rows: int, threads: int):
        threads = max(1, min(threads, rows))
        step = -(-rows // threads)
        return [(r0, min(rows, r0 + step)) for r0 in range(0, rows, step)]

    def _run_rows(self, fn, rows: int, threads: int):
        spans = self._split(rows, threads)
        if len(spans) == 1:
            rc = fn(*spans[0])
            if rc != 0:
                raise RuntimeError(f"oracle call failed with status {rc}")
            return
        with ThreadPoolExecutor(max_workers=len(spans)) as pool:
            for rc in pool.map(lambda s: fn(*s), spans):
                if rc != 0:
                    raise RuntimeError(f"oracle call failed with status {rc}")

    # -- softmax -----------------------------------------------------------
    def softmax(self, x: np.ndarray, threads: int = 1) -> np.ndarray:
        """Row-wise softmax in double.  ``x``: 2-D float32, or uint16 bf16 bits."""
        return self._rowwise(x, threads, self.lib.oracle_softmax_f32, self.lib.oracle_softmax_bf16)

    def naive_softmax(self, x: np.ndarray, threads: int = 1) -> np.ndarray:
        """Row-wise e^{x_i} / sum_j e^{x_j} in double, no maximum subtracted."""
        return self._rowwise(x, threads, self.lib.oracle_naive_softmax_f32, self.lib.oracle_naive_softmax_bf16)

    def _rowwise(self, x: np.ndarray, threads: int, fn32, fn16) -> np.ndarray:
        x = np.ascontiguousarray(x)
        if x.ndim != 2:
            raise ValueError("x must be 2-D [rows, cols]")
        rows, cols = x.shape
        y = np.empty((rows, cols), dtype=np.float64)
        if rows == 0 or cols == 0:
            return y
        if x.dtype == np.float32:
            fn, esz = fn32, 4
        elif x.dtype == np.uint16:
            fn, esz = fn16, 2
        else:
            raise TypeError("x must be float32 or uint16 (bf16 bit patterns)")
        xb, yb = x.ctypes.data, y.ctypes.data

        def part(r0, r1):
            return fn(ctypes.c_void_p(xb + r0 * cols * esz), r1 - r0, cols,
                      ctypes.c_void_p(yb + r0 * cols * 8))

        self._run_rows(part, rows, threads)
        return y

    def stats(self, x: np.ndarray, threads: int = 1):
        """Per-row (m, d) in double by the plain definition."""
        x = np.ascontiguousarray(x)
        rows, cols = x.shape
        m = np.empty(rows, dtype=np.float64)
        d = np.empty(rows, dtype=np.float64)
        if rows == 0:
            return m, d
        if x.dtype == np.float32:
            fn, esz = self.lib.oracle_stats_f32, 4
        elif x.dtype == np.uint16:
            fn, esz = self.lib.oracle_stats_bf16, 2
        else:
            raise TypeError("x must be float32 or uint16 (bf16 bit patterns)")
        xb, mb, db = x.ctypes.data, m.ctypes.data, d.ctypes.data

        def part(r0, r1):
            return fn(ctypes.c_void_p(xb + r0 * cols * esz), r1 - r0, cols,
                      ctypes.c_void_p(mb + r0 * 8), ctypes.c_void_p(db + r0 * 8))

        self._run_rows(part, rows, threads)
        return m, d

    def logsumexp(self, x: np.ndarray, threads: int = 1) -> np.ndarray:
        """Per-row log(sum e^{x}) in double."""
        x = np.ascontiguousarray(x)
        rows, cols = x.shape
        out = np.empty(rows, dtype=np.float64)
        if rows == 0:
            return out
        if x.dtype == np.float32:
            fn, esz = self.lib.oracle_logsumexp_f32, 4
        elif x.dtype == np.uint16:
            fn, esz = self.lib.oracle_logsumexp_bf16, 2
        else:
            raise TypeError("x must be float32 or uint16 (bf16 bit patterns)")
        xb, ob = x.ctypes.data, out.ctypes.data

        def part(r0, r1):
            return fn(ctypes.c_void_p(xb + r0 * cols * esz), r1 - r0, cols, ctypes.c_void_p(ob + r0 * 8))

        self._run_rows(part, rows, threads)
        return out

    # -- the recurrence and the operator -------------------------------------
    def online_state(self, x) -> tuple[float, float]:
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1))
        m = ctypes.c_double()
        d = ctypes.c_double()
        self.lib.oracle_online_state(_ptr(x), x.size, ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value

    def combine(self, a, b) -> tuple[float, float]:
        m = ctypes.c_double()
        d = ctypes.c_double()
        self.lib.oracle_combine(float(a[0]), float(a[1]), float(b[0]), float(b[1]),
                                ctypes.byref(m), ctypes.byref(d))
        return m.value, d.value

    # -- fused-softmax top-K, by brute force ----------------------------------
    def topk(self, x: np.ndarray, K: int, threads: int = 1):
        """K best entries per row (value desc, index asc) of a float32 array, or
        of a uint16 array of bf16 bit patterns; probabilities over the whole row."""
        return self._ranked(x, K, threads, self.lib.oracle_topk_f32, self.lib.oracle_topk_bf16)

    def topk_select(self, x: np.ndarray, K: int, threads: int = 1):
        """K best entries per row (value desc, index asc), returned as the
        entries themselves (in double) with their columns."""
        return self._ranked(x, K, threads, self.lib.oracle_topk_select_f32, self.lib.oracle_topk_select_bf16)

    def _ranked(self, x: np.ndarray, K: int, threads: int, fn32, fn16):
        x = np.ascontiguousarray(x)
        if x.dtype == np.float32:
            fn, esz = fn32, 4
        elif x.dtype == np.uint16:
            fn, esz = fn16, 2
        else:
            raise TypeError("x must be float32 or uint16 (bf16 bit patterns)")
        rows, cols = x.shape
        probs = np.empty((rows, K), dtype=np.float64)
        idx = np.empty((rows, K), dtype=np.int32)
        if rows == 0:
            return probs, idx
        xb, pb, ib = x.ctypes.data, probs.ctypes.data, idx.ctypes.data

        def part(r0, r1):
            return fn(ctypes.c_void_p(xb + r0 * cols * esz), r1 - r0, cols, K,
                      ctypes.c_void_p(pb + r0 * K * 8), ctypes.c_void_p(ib + r0 * K * 4))

        self._run_rows(part, rows, threads)
        return probs, idx


    # -- attention -----------------------------------------------------------
    @staticmethod
    def _attn_args(q, k, v, causal, q_off):
        q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
        for a in (q, k, v):
            if a.dtype != np.uint16 or a.ndim != 3:
                raise TypeError("q, k, v must be uint16 (bf16 bit patterns) of shape [heads, n, d]")
        heads, nq, d = q.shape
        if k.shape != v.shape or k.shape[0] != heads or k.shape[2] != d:
            raise ValueError("k and v must be [heads, nk, d] with q's heads and d")
        if causal and q_off + nq > k.shape[1]:
            raise ValueError("causal attention needs q_off + nq <= nk")
        return q, k, v, heads, nq, k.shape[1], d

    def attention(self, q, k, v, scale: float, causal: bool = False, q_off: int = 0, threads: int = 1,
                  want_abs: bool = False):
        """(O, L[, O_abs]) in double: O [heads, nq, d], L [heads, nq]; q holds
        query rows q_off .. q_off + nq - 1 of each head.  O_abs = the same
        weights applied to |V|."""
        q, k, v, heads, nq, nk, d = self._attn_args(q, k, v, causal, q_off)
        o = np.empty((heads, nq, d), dtype=np.float64)
        lse = np.empty((heads, nq), dtype=np.float64)
        oabs = np.empty((heads, nq, d), dtype=np.float64) if want_abs else None
        fn = self.lib.oracle_attention_bf16

        def part(h0, h1):
            n = h1 - h0
            return fn(ctypes.c_void_p(q[h0:].ctypes.data), ctypes.c_void_p(k[h0:].ctypes.data),
                      ctypes.c_void_p(v[h0:].ctypes.data), n, nq, nk, d, float(scale), int(bool(causal)), q_off,
                      ctypes.c_void_p(o[h0:].ctypes.data), ctypes.c_void_p(lse[h0:].ctypes.data),
                      None if oabs is None else ctypes.c_void_p(oabs[h0:].ctypes.data))

        if heads:
            self._run_rows(part, heads, threads)
        return (o, lse, oabs) if want_abs else (o, lse)

    def attention_tiled(self, q, k, v, scale: float, tile: int, causal: bool = False, q_off: int = 0):
        q, k, v, heads, nq, nk, d = self._attn_args(q, k, v, causal, q_off)
        o = np.empty((heads, nq, d), dtype=np.float64)
        lse = np.empty((heads, nq), dtype=np.float64)
        rc = self.lib.oracle_attention_tiled_bf16(_ptr(q), _ptr(k), _ptr(v), heads, nq, nk, d, float(scale),
                                                  int(bool(causal)), q_off, tile, _ptr(o), _ptr(lse))
        if rc != 0:
            raise RuntimeError(f"oracle call failed with status {rc}")
        return o, lse


_DEFAULT: Oracle | None = None


def load(path: str = DEFAULT_LIB) -> Oracle:
    """The oracle built from ``oracle/oracle.c`` (cached)."""
    global _DEFAULT
    if path != DEFAULT_LIB:
        return Oracle(path)
    if _DEFAULT is None:
        _DEFAULT = Oracle(path)
    return _DEFAULT
