"""Q4_0 matmul oracle (TEST INFRASTRUCTURE ONLY).

A thin ctypes front end to ``q4_0_oracle.c``: a plain CPU dequantize-to-fp32,
accumulate-in-fp64 implementation of y = x . W^T for W stored as GGUF Q4_0
blocks.  Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library in ``gemm_q4_amd`` and neither imports the other.

The C file's header states what the oracle follows and how it is pinned.
The Python helpers here are pinned as follows (tests/test_oracle_pins.py;
tests/test_oracle_mutants.py plants a mistake in each and checks that a pin
fails):

- max_ratio: hand-worked cases (a per-output ratio that a norm-wise ratio
  would under-report, the absolute value, den = 0 with y = 0 and y != 0,
  NaN and Inf outputs, all-zero inputs, the maximum over rows) and a plain
  loop over the outputs on random data;
- greedy_pick: hand-worked ties, NaN and all-NaN rows, and a brute-force
  scan on random integer logits;
- pick_within_tolerance: a near tie inside the two outputs' error budget,
  a far value and an invalid index outside it, and a case that only a
  two-sided budget accepts.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

class Oracle:
    """The oracle's C functions, loaded from one shared library build."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.q4o_half_to_float.argtypes = [ctypes.c_uint16]
        lib.q4o_half_to_float.restype = ctypes.c_float
        lib.q4o_dequantize.argtypes = [vp, i64, i64, vp]
        lib.q4o_dequantize.restype = ctypes.c_int
        lib.q4o_matmul_rows.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64,
                                        vp, i64, vp, vp, ctypes.c_int]
        lib.q4o_matmul_rows.restype = ctypes.c_int
        lib.q4o_quantize_x8.argtypes = [vp, i64, i64, vp, vp]
        lib.q4o_quantize_x8.restype = ctypes.c_int
        lib.q4o_matmul_w4a8_rows.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp, vp,
                                             ctypes.c_int]
        lib.q4o_matmul_w4a8_rows.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def half_to_float(self, bits: int) -> float:
        """Decode one binary16 bit pattern with the oracle's own decoder."""
        return float(self.lib.q4o_half_to_float(bits & 0xFFFF))

    def dequantize(self, blocks: np.ndarray, out: int, in_: int) -> np.ndarray:
        """[out x in] float32 weights d*(q-8) from uint8 GGUF Q4_0 blocks."""
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        if in_ % 32 or blocks.size != out * (in_ // 32) * 18:
            raise ValueError("block buffer does not match out x in")
        w = np.empty((out, in_), dtype=np.float32)
        if self.lib.q4o_dequantize(_ptr(blocks), out, in_, _ptr(w)) != 0:
            raise ValueError("oracle rejected the shape")
        return w

    def matmul(self, blocks: np.ndarray, x: np.ndarray, out: int, in_: int,
               rows=None, nthreads: int = 0, return_threads: bool = False):
        """Return (y, den), float64 [n x len(rows)] (all rows when rows is None).

        y[t, i] = sum_k w[o, k] x[t, k] with o = rows[i];
        den[t, i] = sum_k |w[o, k] x[t, k]|.
        x is float32 or float16, [n x in].
        """
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        if in_ % 32 or blocks.size != out * (in_ // 32) * 18:
            raise ValueError("block buffer does not match out x in")
        if x.dtype == np.float16:
            xa, is16 = np.ascontiguousarray(x).view(np.uint16), 1
        elif x.dtype == np.float32:
            xa, is16 = np.ascontiguousarray(x), 0
        else:
            raise TypeError("x must be float32 or float16")
        if xa.ndim != 2 or xa.shape[1] != in_:
            raise ValueError("x must be [n x in]")
        n = xa.shape[0]
        if rows is None:
            nrows, rp = out, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nrows, rp = rows_arr.size, _ptr(rows_arr)
        y = np.empty((n, nrows), dtype=np.float64)
        den = np.empty((n, nrows), dtype=np.float64)
        rc = self.lib.q4o_matmul_rows(_ptr(blocks), _ptr(xa), is16, n, out,
                                      in_, rp, nrows, _ptr(y), _ptr(den),
                                      nthreads)
        if rc < 0:
            raise ValueError(f"oracle failed with status {rc}")
        return (y, den, rc) if return_threads else (y, den)


    def quantize_x8(self, x: np.ndarray):
        """(q int8 [n x in], d float32 [n x in/32]): x quantized per 32-value
        block (see q4o_quantize_x8)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        n, in_ = x.shape
        q = np.empty((n, in_), dtype=np.int8)
        d = np.empty((n, in_ // 32), dtype=np.float32)
        if self.lib.q4o_quantize_x8(_ptr(x), n, in_, _ptr(q), _ptr(d)) != 0:
            raise ValueError("oracle rejected the shape")
        return q, d

    def matmul_w4a8(self, blocks: np.ndarray, q: np.ndarray, d: np.ndarray, out: int,
                    in_: int, rows=None, nthreads: int = 0):
        """(y, den) float64 [n x len(rows)] of the W4A8 product on quantized
        activations (q, d) (see q4o_matmul_w4a8_rows)."""
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        q = np.ascontiguousarray(q, dtype=np.int8)
        d = np.ascontiguousarray(d, dtype=np.float32)
        if in_ % 32 or blocks.size != out * (in_ // 32) * 18:
            raise ValueError("block buffer does not match out x in")
        n = q.shape[0]
        if q.shape != (n, in_) or d.shape != (n, in_ // 32):
            raise ValueError("q must be [n x in] and d [n x in/32]")
        if rows is None:
            nrows, rp = out, None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nrows, rp = rows_arr.size, _ptr(rows_arr)
        y = np.empty((n, nrows), dtype=np.float64)
        den = np.empty((n, nrows), dtype=np.float64)
        rc = self.lib.q4o_matmul_w4a8_rows(_ptr(blocks), _ptr(q), _ptr(d), n, out, in_, rp,
                                          nrows, _ptr(y), _ptr(den), nthreads)
        if rc < 0:
            raise ValueError(f"oracle failed with status {rc}")
        return y, den


_DEFAULT = None


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default() -> Oracle:
    """The oracle built from ``q4_0_oracle.c`` (compiled on first use)."""
    global _DEFAULT
    if _DEFAULT is None:
        path = _build.LIB
        if not os.path.exists(path) or (
                os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        _DEFAULT = Oracle(path)
    return _DEFAULT


def half_to_float(bits: int) -> float:
    return default().half_to_float(bits)


def dequantize(blocks, out, in_):
    return default().dequantize(blocks, out, in_)


def matmul(blocks, x, out, in_, rows=None, nthreads=0, return_threads=False):
    return default().matmul(blocks, x, out, in_, rows, nthreads, return_threads)


def quantize_x8(x):
    return default().quantize_x8(x)


def matmul_w4a8(blocks, q, d, out, in_, rows=None, nthreads=0):
    return default().matmul_w4a8(blocks, q, d, out, in_, rows, nthreads)


def max_ratio(y: np.ndarray, y_ref: np.ndarray, den: np.ndarray) -> float:
    """Acceptance metric: max over outputs of |y - y_ref| / den.

    Where den == 0 every product is zero, so y must be exactly 0 there; any
    other value counts as an infinite ratio.
    """
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    zero = den == 0
    if np.any(zero & (y != 0)):
        return float("inf")
    if np.any(~np.isfinite(y[~zero])):
        return float("inf")
    if not np.any(~zero):
        return 0.0
    return float(np.max(err[~zero] / den[~zero]))


def greedy_pick(y_ref: np.ndarray):
    """The greedy pick of a logit head (golem README, "Several conversations,
    one pass": the output head scores every state of a pass): per row t of
    y_ref, the largest value and its index, the smallest index among equal
    values.  A plain scan, written out so ties and NaN are explicit: a NaN
    never wins; a row with no number gives (nan, -1)."""
    y_ref = np.asarray(y_ref, dtype=np.float64)
    vals, idxs = [], []
    for row in y_ref:
        best, bi = -np.inf, -1
        for i, v in enumerate(row.tolist()):
            if v > best or (v == best and bi < 0):
                best, bi = v, i
        vals.append(best if bi >= 0 else np.nan)
        idxs.append(bi)
    return np.array(vals, dtype=np.float64), np.array(idxs, dtype=np.int64)


def pick_within_tolerance(y_ref: np.ndarray, den: np.ndarray, idx: np.ndarray,
                          tol: float) -> bool:
    """Whether idx[t] is a correct pick for every row t given outputs that may
    each be off by up to tol * den: y_ref[t, idx] is within the two outputs'
    error budgets of the row's true maximum (several indices can be correct
    when logits nearly tie)."""
    best, bi = greedy_pick(y_ref)
    for t, i in enumerate(np.asarray(idx).tolist()):
        if i < 0 or i >= y_ref.shape[1]:
            return False
        slack = tol * (den[t, i] + den[t, bi[t]])
        if y_ref[t, i] < best[t] - slack:
            return False
    return True
