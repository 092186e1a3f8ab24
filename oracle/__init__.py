"""CPU oracle for SGMV expand-slice and its LoRA-A projection -- TEST
INFRASTRUCTURE ONLY.

A ctypes binding over ``libsgmv_oracle.so`` (plain C, fp64, see
``sgmv_oracle.h``).  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package; the GPU library never
does, and this package never imports the GPU library.

What it computes (wiki page "Implementation: Predibase Lorax SGMV Expand
Slice Kernel", Description and I/O Contract): for every segment b with
adapter a = idx[b] != -1 and every row t in [start_b, start_b + len_b),

    out[t][off + n] = rne( (add ? out0[t][off + n] : 0) + sum_k x[t][k] * W[a][n][k] )

in fp64 with a single round-to-nearest-even into the output dtype; every
other element of ``out`` keeps its bits.  float32 inputs are first rounded
to the 16-bit weight dtype (the page's CAST_TYPE mixed-precision cast).

``shrink`` is the LoRA-A projection that produces the expand's inputs (the
page describes them as that projection's low-rank activations):
``y[t][k] = rne(scale * sum_h x[t][h] * A[a][k][h])`` for rows of active
segments, lora_A stacked (lora_num, rank, hidden); see ``sgmv_oracle.h``
for the readings it takes where the page is silent.

``fused`` is the two composed: ``shrink`` into outputs of the weights'
16-bit dtype, then ``expand`` of those outputs (the fused LoRA delta of a
QKV or gate/up layer); it adds no arithmetic of its own.

Arrays are numpy: 16-bit storage as ``uint16`` bit patterns, float32 as
``float32``.  Dtype names are "f16", "bf16", "f32".
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY names another build of sgmv_oracle.c (the mutation test
# loads deliberately broken copies to show that the pins catch them).
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "libsgmv_oracle.so")

DTYPE_CODES = {"f16": 0, "bf16": 1, "f32": 2}
_STORAGE = {"f16": np.uint16, "bf16": np.uint16, "f32": np.float32}

OK, BAD_ARGUMENT, BAD_SEGMENT, BAD_INDEX, NO_MEMORY = range(5)


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        names = {1: "bad argument", 2: "bad segment", 3: "bad adapter index", 4: "out of memory"}
        super().__init__(f"oracle {what}: {names.get(code, code)}")
        self.code = code


class _Slice(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("x_stride", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("w_dtype", ctypes.c_int), ("N", ctypes.c_int64),
                ("offset", ctypes.c_int64)]


class _ShrinkSlice(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("out", ctypes.c_void_p), ("out_stride", ctypes.c_int64)]


class _Report(ctypes.Structure):
    _fields_ = [("checked_values", ctypes.c_int64), ("checked_untouched", ctypes.c_int64),
                ("bad_values", ctypes.c_int64), ("bad_untouched", ctypes.c_int64),
                ("max_abs_err", ctypes.c_double), ("max_tol_ratio", ctypes.c_double),
                ("first_bad_row", ctypes.c_int64), ("first_bad_col", ctypes.c_int64)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        p, i64, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_decode.argtypes = [i, ctypes.c_uint32]
        lib.orc_decode.restype = ctypes.c_double
        lib.orc_encode.argtypes = [i, ctypes.c_double]
        lib.orc_encode.restype = ctypes.c_uint32
        lib.orc_decode_array.argtypes = [i, p, p, i64]
        lib.orc_encode_array.argtypes = [i, p, p, i64]
        lib.orc_expand.argtypes = [p, i, i64, i64, p, i, i64, i64, i64, p, p, p, i64, i, p, i]
        lib.orc_expand.restype = i
        lib.orc_check.argtypes = [p, i, i64, i64, p, p, i, i64, i64, i64, p, p, p, i64, i,
                                  ctypes.c_double, ctypes.c_double, p, i64, i, p]
        lib.orc_check.restype = i
        lib.orc_shrink.argtypes = [p, i, i64, i64, i64, p, i, i, i64, i64, i, p, p, p, i64,
                                   ctypes.c_double, p, i64, p, i]
        lib.orc_shrink.restype = i
        lib.orc_threads.argtypes = [i]
        lib.orc_threads.restype = i
        _lib = lib
    return _lib


@dataclass
class Slice:
    """One slice: inputs x (T, >=K) with row stride, weights w (L, N, K), offset."""
    x: np.ndarray
    x_dtype: str
    w: np.ndarray
    w_dtype: str
    offset: int

    @property
    def N(self) -> int:
        return int(self.w.shape[1])


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_storage(a: np.ndarray, dtype: str, what: str):
    if a.dtype != _STORAGE[dtype]:
        raise TypeError(f"{what}: expected {np.dtype(_STORAGE[dtype])} storage for {dtype}, got {a.dtype}")


def _slices(slices: Sequence[Slice], K: int, L: int):
    arr = (_Slice * len(slices))()
    keep = []
    for i, s in enumerate(slices):
        _check_storage(s.x, s.x_dtype, "x")
        _check_storage(s.w, s.w_dtype, "w")
        if s.x.ndim != 2 or s.x.strides[1] != s.x.itemsize:
            raise ValueError("x must be 2-D with unit column stride")
        w = np.ascontiguousarray(s.w)
        if w.shape[0] != L or w.shape[2] != K:
            raise ValueError(f"w shape {w.shape} does not match L={L}, K={K}")
        keep.append(w)
        arr[i] = _Slice(_ptr(s.x), DTYPE_CODES[s.x_dtype], s.x.strides[0] // s.x.itemsize,
                        _ptr(w), DTYPE_CODES[s.w_dtype], w.shape[1], s.offset)
    return arr, keep


def _meta(start, lens, idx):
    start = np.ascontiguousarray(start, dtype=np.int64)
    lens = np.ascontiguousarray(lens, dtype=np.int64)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    if not (start.shape == lens.shape == idx.shape) or start.ndim != 1:
        raise ValueError("segment metadata must be three 1-D arrays of equal length")
    return start, lens, idx


def decode(dtype: str, bits: np.ndarray) -> np.ndarray:
    """Exact fp64 values of stored bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(b.shape, dtype=np.float64)
    _load().orc_decode_array(DTYPE_CODES[dtype], _ptr(b), _ptr(out), b.size)
    return out


def encode(dtype: str, values: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even bit patterns (uint32) of fp64 values."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint32)
    _load().orc_encode_array(DTYPE_CODES[dtype], _ptr(v), _ptr(out), v.size)
    return out


def threads(requested: int = 0) -> int:
    """Threads an oracle call with ``threads=requested`` uses."""
    return _load().orc_threads(requested)


def expand(slices: Sequence[Slice], out: np.ndarray, out_dtype: str,
           start, lens, idx, add_inputs: bool, K: int, L: int,
           want_ref: bool = False, threads: int = 0) -> Optional[list]:
    """Apply the slices to ``out`` (holding O0) in place.

    Returns, if ``want_ref``, one (T, N_s) fp64 array per slice holding the
    exact pre-rounding values (NaN where the row is not in an active segment).
    """
    lib = _load()
    _check_storage(out, out_dtype, "out")
    if out.ndim != 2 or out.strides[1] != out.itemsize:
        raise ValueError("out must be 2-D with unit column stride")
    start, lens, idx = _meta(start, lens, idx)
    arr, keep = _slices(slices, K, L)
    T, H = out.shape
    ref = None
    if want_ref:
        ref = np.full(sum(T * s.N for s in slices), np.nan, dtype=np.float64)
    rc = lib.orc_expand(arr, len(slices), K, L, _ptr(out), DTYPE_CODES[out_dtype], T, H,
                        out.strides[0] // out.itemsize, _ptr(start), _ptr(lens), _ptr(idx),
                        len(start), int(bool(add_inputs)), _ptr(ref) if want_ref else None,
                        threads)
    del keep
    if rc != OK:
        raise OracleError(rc, "expand")
    if not want_ref:
        return None
    views, base = [], 0
    for s in slices:
        views.append(ref[base:base + T * s.N].reshape(T, s.N))
        base += T * s.N
    return views


def bgmv_expand(slices: Sequence[Slice], out: np.ndarray, out_dtype: str, idx,
                add_inputs: bool, K: int, L: int, want_ref: bool = False,
                threads: int = 0) -> Optional[list]:
    """The per-token counterpart that the page's Description names (BGMV
    expand slice): row t takes adapter idx[t], -1 leaves it untouched.  It is
    the same definition with row t alone as segment t (start t, length 1)."""
    T = out.shape[0]
    return expand(slices, out, out_dtype, np.arange(T, dtype=np.int64),
                  np.ones(T, dtype=np.int64), idx, add_inputs, K, L, want_ref, threads)


@dataclass
class Report:
    checked_values: int
    checked_untouched: int
    bad_values: int
    bad_untouched: int
    max_abs_err: float
    max_tol_ratio: float
    first_bad: Optional[tuple]

    @property
    def ok(self) -> bool:
        return self.bad_values == 0 and self.bad_untouched == 0


def check(slices: Sequence[Slice], prior: np.ndarray, cand: np.ndarray, out_dtype: str,
          start, lens, idx, add_inputs: bool, K: int, L: int, atol: float, rtol: float,
          rows: Optional[np.ndarray] = None, threads: int = 0) -> Report:
    """Stream-compare a candidate output with the exact result (see orc_check)."""
    lib = _load()
    _check_storage(prior, out_dtype, "prior")
    _check_storage(cand, out_dtype, "cand")
    if prior.shape != cand.shape or prior.strides != cand.strides or prior.ndim != 2:
        raise ValueError("prior and cand must be 2-D arrays of the same shape and layout")
    start, lens, idx = _meta(start, lens, idx)
    arr, keep = _slices(slices, K, L)
    T, H = prior.shape
    rows_arr = None
    if rows is not None:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
    rep = _Report()
    rc = lib.orc_check(arr, len(slices), K, L, _ptr(prior), _ptr(cand), DTYPE_CODES[out_dtype],
                       T, H, prior.strides[0] // prior.itemsize, _ptr(start), _ptr(lens),
                       _ptr(idx), len(start), int(bool(add_inputs)), atol, rtol,
                       _ptr(rows_arr) if rows_arr is not None else None,
                       len(rows_arr) if rows_arr is not None else 0, threads, ctypes.byref(rep))
    del keep
    if rc != OK:
        raise OracleError(rc, "check")
    first = None if rep.first_bad_row < 0 else (rep.first_bad_row, rep.first_bad_col)
    return Report(rep.checked_values, rep.checked_untouched, rep.bad_values, rep.bad_untouched,
                  rep.max_abs_err, rep.max_tol_ratio, first)


def shrink(x: np.ndarray, x_dtype: str, lora_a: Sequence[np.ndarray], a_dtype: str,
           outs: Sequence[np.ndarray], out_dtype: str, start, lens, idx, scale: float = 1.0,
           rows: Optional[np.ndarray] = None, want_ref: bool = False,
           threads: int = 0) -> Optional[list]:
    """LoRA-A projection into ``outs`` (one (T, K) array per lora_A stack
    (L, K, H)), in place: row t of an active segment with adapter a gets
    ``rne(scale * sum_h x[t][h] * A[a][k][h])``; other rows keep their bits
    (see orc_shrink for the readings).  ``rows`` restricts the work to those
    rows.  Returns, if ``want_ref``, one (T, K) fp64 array per slice of the
    exact pre-rounding values (NaN where not computed)."""
    lib = _load()
    _check_storage(x, x_dtype, "x")
    if x.ndim != 2 or x.strides[1] != x.itemsize:
        raise ValueError("x must be 2-D with unit column stride")
    T, H = x.shape
    if len(lora_a) != len(outs) or not lora_a:
        raise ValueError("one output per lora_A stack")
    keep = [np.ascontiguousarray(a) for a in lora_a]
    L, K = keep[0].shape[0], keep[0].shape[1]
    arr = (_ShrinkSlice * len(keep))()
    for i, (a, o) in enumerate(zip(keep, outs)):
        _check_storage(a, a_dtype, "lora_a")
        _check_storage(o, out_dtype, "out")
        if a.shape != (L, K, H):
            raise ValueError(f"lora_a shape {a.shape} is not ({L}, {K}, {H})")
        if o.ndim != 2 or o.shape != (T, K) or o.strides[1] != o.itemsize:
            raise ValueError(f"out must be ({T}, {K}) with unit column stride")
        arr[i] = _ShrinkSlice(_ptr(a), _ptr(o), o.strides[0] // o.itemsize)
    start, lens, idx = _meta(start, lens, idx)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    ref = np.full(len(keep) * T * K, np.nan, dtype=np.float64) if want_ref else None
    rc = lib.orc_shrink(_ptr(x), DTYPE_CODES[x_dtype], x.strides[0] // x.itemsize, T, H, arr,
                        len(keep), DTYPE_CODES[a_dtype], K, L, DTYPE_CODES[out_dtype],
                        _ptr(start), _ptr(lens), _ptr(idx), len(start), float(scale),
                        _ptr(rows_arr) if rows_arr is not None else None,
                        len(rows_arr) if rows_arr is not None else 0,
                        _ptr(ref) if want_ref else None, threads)
    del keep
    if rc != OK:
        raise OracleError(rc, "shrink")
    if not want_ref:
        return None
    return [ref[i * T * K:(i + 1) * T * K].reshape(T, K) for i in range(len(outs))]


def fused(x: np.ndarray, x_dtype: str, lora_a: Sequence[np.ndarray],
          lora_b: Sequence[np.ndarray], w_dtype: str, offsets: Sequence[int], out: np.ndarray,
          out_dtype: str, start, lens, idx, scale: float, add_inputs: bool,
          want_ref: bool = False, threads: int = 0):
    """The fused LoRA delta, in place on ``out``: for each slice s, the
    projection y_s = shrink(x, lora_a[s]) rounded to ``w_dtype`` (the
    weights' dtype), then expand(y_s, lora_b[s]) into the window at
    offsets[s].  Returns (the projections, one (T, K) ``w_dtype`` array per
    slice -- zero in rows without an adapter -- and, if ``want_ref``, the
    expand's exact values per slice as ``expand`` returns them)."""
    T = x.shape[0]
    L, K = lora_a[0].shape[0], lora_a[0].shape[1]
    ys = [np.zeros((T, K), dtype=_STORAGE[w_dtype]) for _ in lora_a]
    shrink(x, x_dtype, lora_a, w_dtype, ys, w_dtype, start, lens, idx, scale, threads=threads)
    slices = [Slice(y, w_dtype, np.ascontiguousarray(b), w_dtype, int(off))
              for y, b, off in zip(ys, lora_b, offsets)]
    ref = expand(slices, out, out_dtype, start, lens, idx, add_inputs, K, L, want_ref=want_ref,
                 threads=threads)
    return ys, ref


def fused_slices(ys: Sequence[np.ndarray], lora_b: Sequence[np.ndarray], w_dtype: str,
                 offsets: Sequence[int]):
    """The expand slices of a fused call, given its projections (for
    ``check``)."""
    return [Slice(y, w_dtype, np.ascontiguousarray(b), w_dtype, int(off))
            for y, b, off in zip(ys, lora_b, offsets)]
