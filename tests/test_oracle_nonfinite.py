"""Pins of the oracle on non-finite results (IEEE 754 propagation in rows of
active segments) and of its comparator's branch for exact values that are
not finite: NaN where an input, weight or prior value is NaN or a product is
Inf * 0 or a sum meets +Inf and -Inf; +-Inf where an Inf term meets only
finite ones or the exact value lies at or beyond the output format's
overflow threshold (round to nearest even: 65520 and above is +Inf in f16).

The expected classes and values come from numpy's element-wise IEEE
arithmetic in float64 and numpy's correctly rounded float16 / float32 casts,
not from the oracle."""
import numpy as np
import pytest

import oracle
import sgmv_workloads as W
from oracle_pins_util import np_cast_input, np_values, row_adapters

TOL = {"f16": (1e-3, 2e-3), "f32": (1e-5, 1e-5), "bf16": (1e-3, 8e-3)}


def oracle_run(wl):
    s = wl.slices[0]
    out = wl.out0.copy()
    ref = oracle.expand([oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset)], out,
                        wl.out_dtype, wl.start, wl.lens, wl.idx, wl.add, wl.K, wl.L,
                        want_ref=True)[0]
    return out, ref


def elementwise_reference(wl):
    """Exact values of the written window, element by element in float64
    (no BLAS: products summed with numpy's IEEE add), and the written rows."""
    s = wl.slices[0]
    ra = row_adapters(wl)
    xv = np_cast_input(np.ascontiguousarray(s.x), s.x_dtype, s.w_dtype)
    wv = np_values(s.w, s.w_dtype)
    prior = np_values(np.ascontiguousarray(wl.out0[:, s.offset:s.offset + s.N]), wl.out_dtype)
    exp = np.full((wl.T, s.N), np.nan)
    with np.errstate(invalid="ignore", over="ignore"):
        for t in np.nonzero(ra >= 0)[0]:
            acc = prior[t].copy() if wl.add else np.zeros(s.N)
            for k in range(wl.K):
                acc = acc + xv[t, k] * wv[ra[t], :, k]
            exp[t] = acc
    return exp, ra >= 0


def encode_np(v, dtype):
    with np.errstate(over="ignore", invalid="ignore"):
        if dtype == "f16":
            return v.astype(np.float16).view(np.uint16)
        return v.astype(np.float32)


def check(wl, cand):
    s = wl.slices[0]
    atol, rtol = TOL[wl.out_dtype]
    return oracle.check([oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset)], wl.out0, cand,
                        wl.out_dtype, wl.start, wl.lens, wl.idx, wl.add, wl.K, wl.L, atol, rtol)


@pytest.mark.parametrize("dts", [("f16", "f16", "f16"), ("f32", "f16", "f32"),
                                 ("f32", "f16", "f16")])
@pytest.mark.parametrize("add", [False, True])
def test_nonfinite_values_follow_ieee(dts, add):
    wl = W.nonfinite(*dts, add=add)
    out, ref = oracle_run(wl)
    exp, rows = elementwise_reference(wl)
    s = wl.slices[0]
    # exact values: the same NaN positions, the same infinities, the same finite values
    assert np.array_equal(np.isnan(ref[rows]), np.isnan(exp[rows]))
    fin = ~np.isnan(exp[rows])
    assert np.array_equal(ref[rows][fin], exp[rows][fin])
    # every planted kind of value occurs
    assert np.isnan(exp[1]).all()                          # NaN input
    assert np.isposinf(exp[2]).any() and np.isneginf(exp[2]).any() and np.isnan(exp[2]).any()
    assert np.isnan(exp[3]).any()                          # +Inf - Inf
    assert np.isnan(exp[6:11, 5]).all()                    # NaN weight
    assert np.isinf(exp[6:11, 9]).any()                    # Inf weight
    if add:
        assert np.isneginf(exp[4, 5]) and np.isnan(exp[5, 7])
    else:
        assert np.isfinite(exp[4, 5]) and np.isfinite(exp[5, 7])
    if dts[0] == "f32":
        assert not np.isfinite(exp[17]).any()              # input cast overflows to +Inf
    # the rounded output: numpy's correctly rounded cast of the exact value
    win = out[:, s.offset:s.offset + s.N]
    enc = encode_np(exp, wl.out_dtype)
    nan_exp = np.isnan(exp)
    got_vals = np_values(np.ascontiguousarray(win), wl.out_dtype)
    assert np.array_equal(np.isnan(got_vals[rows]), nan_exp[rows])
    assert np.array_equal(win[rows][~nan_exp[rows]], enc[rows][~nan_exp[rows]])
    assert np.isnan(np_values(np.ascontiguousarray(win[rows][nan_exp[rows]]), wl.out_dtype)).all()
    if wl.out_dtype == "f16":
        # the overflow row: |sum| * 6144 at or above 65520 rounds to +-Inf
        assert np.isinf(got_vals[16]).any() and np.isfinite(got_vals[16]).any()
        assert np.array_equal(np.isinf(got_vals[16]), np.abs(exp[16]) >= 65520)
    # rows of the index -1 segment (with their planted NaNs) keep their bits
    bits = (lambda a: a.view(np.uint32)) if wl.out_dtype == "f32" else (lambda a: a)
    assert np.array_equal(bits(out[11:15]), bits(wl.out0[11:15]))
    assert check(wl, out).ok


def test_f16_overflow_threshold_rounds_to_nearest_even():
    """65504 + 15 stays 65504; 65504 + 16 = 65520, the midpoint to the first
    value past the largest finite f16, rounds to even, i.e. +Inf."""
    wl = W.custom([1], [0], K=8, N=2, H=2, off=0, L=1, x_dtype="f16", w_dtype="f16",
                  out_dtype="f16", add=True, values="int", seed=1)
    s = wl.slices[0]
    x = np.array([[1, 0, 0, 0, 0, 0, 0, 0]], dtype=np.float16).view(np.uint16)
    w = np.zeros((1, 2, 8), dtype=np.float16)
    w[0, 0, 0], w[0, 1, 0] = 15, 16
    o = np.array([[65504, 65504]], dtype=np.float16).view(np.uint16)
    wl = W.Workload("edge", [W.SliceInput(x, "f16", w.view(np.uint16), "f16", 0)], o, "f16",
                    wl.start, wl.lens, wl.idx, True, 8, 1)
    out, ref = oracle_run(wl)
    assert ref[0].tolist() == [65519.0, 65520.0]
    assert out[0].view(np.float16).tolist()[0] == 65504.0
    assert np.isposinf(out[0].view(np.float16)[1])


def plant(out, r, c, value, dtype):
    bad = out.copy()
    if dtype == "f16":
        bad[r, c] = np.array([value], dtype=np.float16).view(np.uint16)[0]
    else:
        bad[r, c] = np.float32(value)
    return bad


def test_comparator_nonfinite_branch_catches_planted_mistakes():
    wl = W.nonfinite("f16", "f16", "f16", add=True)
    out, ref = oracle_run(wl)
    off = wl.slices[0].offset
    assert check(wl, out).ok
    vals = out.view(np.float16)
    pinf = [(r, c) for r in range(wl.T) for c in range(off, off + 64)
            if np.isposinf(vals[r, c]) and np.isposinf(ref[r, c - off])]
    ninf = [(r, c) for r in range(wl.T) for c in range(off, off + 64) if np.isneginf(vals[r, c])]
    nans = [(r, c) for r in range(wl.T) for c in range(off, off + 64)
            if np.isnan(vals[r, c]) and r not in range(11, 15)]
    over = [(16, c) for c in range(off, off + 64)
            if np.isposinf(vals[16, c]) and np.isfinite(ref[16, c - off])]
    assert pinf and ninf and nans and over

    def one_bad(cand, where):
        rep = check(wl, cand)
        assert rep.bad_values == 1 and rep.bad_untouched == 0 and rep.first_bad == where, rep

    r, c = pinf[0]
    one_bad(plant(out, r, c, -np.inf, "f16"), (r, c))      # wrong sign
    one_bad(plant(out, r, c, 65504.0, "f16"), (r, c))      # largest finite value
    one_bad(plant(out, r, c, np.nan, "f16"), (r, c))       # NaN for Inf
    r, c = ninf[0]
    one_bad(plant(out, r, c, np.inf, "f16"), (r, c))
    r, c = nans[0]
    one_bad(plant(out, r, c, np.inf, "f16"), (r, c))       # Inf for NaN
    one_bad(plant(out, r, c, 0.0, "f16"), (r, c))          # finite for NaN
    other_nan = out.copy()
    other_nan[r, c] = 0x7E01 if out[r, c] != 0x7E01 else 0x7E02   # any NaN is a NaN
    assert check(wl, other_nan).ok
    r, c = over[0]                                          # exact value finite, rounds to +Inf
    one_bad(plant(out, r, c, 65504.0, "f16"), (r, c))
    r, c = 0, off                                           # finite value, Inf candidate
    assert np.isfinite(vals[r, c])
    one_bad(plant(out, r, c, np.inf, "f16"), (r, c))
    # a NaN planted in an untouched row is a changed untouched element
    bad = plant(out, 12, off, np.nan, "f16")
    rep = check(wl, bad)
    assert rep.bad_untouched == 1 and rep.bad_values == 0


def test_comparator_nonfinite_branch_float32_output():
    wl = W.nonfinite("f32", "f16", "f32", add=False)
    out, ref = oracle_run(wl)
    off = wl.slices[0].offset
    assert check(wl, out).ok
    inf_at = [(17, c) for c in range(off, off + 64) if np.isinf(out[17, c])]
    nan_at = [(17, c) for c in range(off, off + 64) if np.isnan(out[17, c])]
    assert inf_at and nan_at
    r, c = inf_at[0]
    rep = check(wl, plant(out, r, c, -out[r, c], "f32"))
    assert rep.bad_values == 1 and rep.first_bad == (r, c)
    rep = check(wl, plant(out, r, c, 3.4e38 * np.sign(out[r, c]), "f32"))
    assert rep.bad_values == 1
    r, c = nan_at[0]
    rep = check(wl, plant(out, r, c, np.inf, "f32"))
    assert rep.bad_values == 1 and rep.first_bad == (r, c)
