"""Independent references used to pin the oracle (tests only).

Nothing here calls the oracle's arithmetic: stored values are decoded with
numpy views (float16, the upper half of a float32 for bfloat16), float32
inputs are cast with torch's bfloat16 / numpy's float16 conversions, and the
contraction is a numpy matrix product per adapter over a row mask -- a
different formulation from the oracle's per-segment, per-element loops.
"""
import numpy as np


def np_values(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 values of stored data, decoded with numpy only."""
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return a.astype(np.float64)
    raise ValueError(dtype)


def np_cast_input(x: np.ndarray, x_dtype: str, w_dtype: str) -> np.ndarray:
    """Values of the inputs as they enter the products: float32 inputs are
    rounded to the weight dtype by library conversions."""
    if x_dtype != "f32":
        return np_values(x, x_dtype)
    if w_dtype == "f16":
        return x.astype(np.float16).astype(np.float64)
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def row_adapters(wl) -> np.ndarray:
    """Adapter applied to each output row (-1: none)."""
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            ra[s:s + n] = a
    return ra


def masked_reference(wl):
    """Expected fp64 output values (whole T x H array) and the boolean mask of
    elements the operation writes, computed as sum over adapters of
    (rows using that adapter) @ W[a]^T."""
    prior = np_values(wl.out0, wl.out_dtype)
    expected = prior.copy()
    written = np.zeros(prior.shape, dtype=bool)
    ra = row_adapters(wl)
    rows = ra >= 0
    for s in wl.slices:
        xv = np_cast_input(np.ascontiguousarray(s.x), s.x_dtype, s.w_dtype)
        wv = np_values(s.w, s.w_dtype)
        y = np.zeros((wl.T, s.N), dtype=np.float64)
        for a in range(wl.L):
            m = ra == a
            if m.any():
                y[m] = xv[m] @ wv[a].T
        cols = slice(s.offset, s.offset + s.N)
        base = prior[:, cols] if wl.add else 0.0
        region = expected[:, cols]
        region[rows] = (base + y)[rows] if wl.add else y[rows]
        written[rows, cols] = True
    return expected, written


def ulp(values: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of representable values of ``dtype`` at |values|."""
    mbits, emin = {"f16": (10, -14), "bf16": (7, -126), "f32": (23, -126)}[dtype]
    a = np.abs(values)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return np.exp2(e - mbits)
