"""Pins for the oracle's LoRA-A projection (shrink) against facts fixed
outside the oracle itself.

The expand page ("Implementation: Predibase Lorax SGMV Expand Slice Kernel",
I/O Contract, Inputs; Usage Examples) describes its ``inputs`` as the
rank-sized activations the A-side LoRA projection produces for every token of
every sequence.  The
readings (lora_A stacked (lora_num, rank, hidden); y = scale * x A[a]^T per
active segment row; float32 inputs rounded to the weight dtype; inactive rows
untouched) are pinned here by

* special cases that reduce to a plain matrix product (numpy BLAS), with
  rank != hidden so a transposed operand cannot pass;
* a per-adapter row-mask formulation over random segments;
* exact integer-valued cases compared bit for bit with numpy integer math;
* the float32-input cast against torch's / numpy's conversions;
* the composition with the expand oracle: shrink then expand equals the
  dense LoRA delta x A^T B^T, exactly, on integer data;
* invariants: scaling, row subsets, multi-slice = separate calls, threads.
"""
import numpy as np
import pytest

import oracle
import sgmv_workloads as W
from oracle_pins_util import np_cast_input, np_values, ulp


def run_shrink(wl, rows=None, want_ref=True, threads=0, scale=None):
    outs = [o.copy() for o in wl.outs0]
    ref = oracle.shrink(wl.x, wl.x_dtype, wl.lora_a, wl.a_dtype, outs, wl.out_dtype, wl.start,
                        wl.lens, wl.idx, wl.scale if scale is None else scale, rows=rows,
                        want_ref=want_ref, threads=threads)
    return outs, ref


def row_adapters(wl):
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            ra[s:s + n] = a
    return ra


def masked_projection(wl, si=0, scale=None):
    """Expected fp64 projection of every row (NaN where no adapter applies):
    for each adapter, (rows using it) @ A[a]^T, times the scale."""
    scale = wl.scale if scale is None else scale
    xv = np_cast_input(np.ascontiguousarray(wl.x), wl.x_dtype, wl.a_dtype)
    av = np_values(wl.lora_a[si], wl.a_dtype)
    ra = row_adapters(wl)
    y = np.full((wl.T, wl.K), np.nan)
    for a in range(wl.L):
        m = ra == a
        if m.any():
            y[m] = (xv[m] @ av[a].T) * scale
    return y


def assert_rounded_from(got_bits, exact, dtype):
    got = np_values(got_bits, dtype)
    assert np.all(np.abs(got - exact) <= 0.5 * ulp(exact, dtype) * (1 + 1e-9) + 1e-300)


# --------------------------------------------------------------------------
# Plain matrix products.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_single_segment_is_a_gemm(out_dtype):
    """One segment over every row with adapter 1: y = rne(x @ A[1]^T)."""
    wl = W.shrink_custom([29], [1], H=72, K=24, L=3, out_dtype=out_dtype, seed=3)
    outs, ref = run_shrink(wl)
    gemm = np_values(wl.x, "bf16") @ np_values(wl.lora_a[0], "bf16")[1].T
    assert np.allclose(ref[0], gemm, rtol=1e-12, atol=1e-13)
    assert_rounded_from(outs[0], gemm, out_dtype)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_segments_match_row_masks(seed):
    """Random lengths (including 0), indices (including -1), shuffled starts
    leaving gaps: written rows match the per-adapter masked products, the
    other rows keep their bits."""
    rng = np.random.default_rng(100 + seed)
    B = 9
    lens = rng.integers(0, 8, size=B)
    idx = rng.integers(-1, 4, size=B)
    gaps = rng.integers(0, 3, size=B)
    order = rng.permutation(B)
    start = np.zeros(B, dtype=np.int64)
    pos = 0
    for b in order:
        pos += int(gaps[b])
        start[b] = pos
        pos += int(lens[b])
    wl = W.shrink_custom(lens, idx, H=56, K=8, L=4, slices=2, x_dtype="f16", a_dtype="f16",
                         out_dtype="f32", start=start, T=pos + 2, scale=0.75, seed=seed)
    outs, ref = run_shrink(wl)
    ra = row_adapters(wl)
    for si in range(2):
        y = masked_projection(wl, si)
        on = ra >= 0
        assert np.allclose(ref[si][on], y[on], rtol=1e-12, atol=1e-13)
        assert np.all(np.isnan(ref[si][~on]))
        assert np.array_equal(outs[si][~on], wl.outs0[si][~on]), "untouched rows changed"
        assert_rounded_from(outs[si][on], y[on], "f32")


# --------------------------------------------------------------------------
# Exact integer-valued cases: x, A in [-3, 3] and hidden 24 give |sum| <= 216,
# an integer that bf16 and fp16 hold exactly; a power-of-two scale keeps it
# exact.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("scale", [1.0, 2.0, 0.25])
@pytest.mark.parametrize("x_dtype,a_dtype,out_dtype", [
    ("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("f32", "bf16", "f32"),
    ("f32", "f16", "bf16"), ("bf16", "bf16", "f32")])
def test_integer_cases_exact(scale, x_dtype, a_dtype, out_dtype):
    wl = W.shrink_custom([3, 0, 6, 4, 5], [1, 0, -1, 0, 2], H=24, K=16, L=3,
                         x_dtype=x_dtype, a_dtype=a_dtype, out_dtype=out_dtype, scale=scale,
                         values="int", seed=11)
    outs, _ = run_shrink(wl)
    x = np_values(np.ascontiguousarray(wl.x), x_dtype).astype(np.int64)
    a = np_values(wl.lora_a[0], a_dtype).astype(np.int64)
    ra = row_adapters(wl)
    expected = wl.outs0[0].copy()
    for t in range(wl.T):
        if ra[t] < 0:
            continue
        r = (x[t] @ a[ra[t]].T).astype(np.float64) * scale
        rf = r.astype(np.float32)
        if out_dtype == "f32":
            expected[t] = rf
        elif out_dtype == "f16":
            expected[t] = rf.astype(np.float16).view(np.uint16)
        else:
            expected[t] = (rf.view(np.uint32) >> 16).astype(np.uint16)  # exact values
    assert np.array_equal(outs[0], expected)


# --------------------------------------------------------------------------
# Float32 inputs are rounded to the weight dtype before the products.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("a_dtype", ["bf16", "f16"])
def test_float32_input_is_cast_to_weight_dtype(a_dtype):
    wl = W.shrink_custom([11, 6], [0, 1], H=40, K=8, L=2, x_dtype="f32", a_dtype=a_dtype,
                         out_dtype="f32", seed=4)
    _, ref = run_shrink(wl)
    xc = np_cast_input(np.ascontiguousarray(wl.x), "f32", a_dtype)
    av = np_values(wl.lora_a[0], a_dtype)
    assert np.allclose(ref[0][:11], xc[:11] @ av[0].T, rtol=1e-12, atol=1e-13)
    assert np.allclose(ref[0][11:], xc[11:] @ av[1].T, rtol=1e-12, atol=1e-13)
    # and it differs from the uncast product (the cast is not a no-op here)
    raw = wl.x.astype(np.float64)
    assert not np.allclose(ref[0][:11], raw[:11] @ av[0].T, rtol=1e-9, atol=0)


# --------------------------------------------------------------------------
# Composition with the expand: the expand's inputs are this projection's
# output (the page's usage example passes lora_a_output as inputs).
# --------------------------------------------------------------------------

def test_shrink_then_expand_is_the_dense_lora_delta():
    """Integer data: shrink into float32, expand (float32 inputs rounded to
    bf16, exact for these integers) onto a zero output: equals
    x @ A[a]^T @ B[a]^T computed with numpy integers, bit for bit."""
    lens, idx = [4, 7, 3, 5], [2, -1, 0, 2]
    H, K, N, L = 20, 8, 24, 3
    sw = W.shrink_custom(lens, idx, H=H, K=K, L=L, x_dtype="bf16", a_dtype="bf16",
                         out_dtype="f32", values="int", seed=21)
    y = [o.copy() for o in sw.outs0]
    oracle.shrink(sw.x, "bf16", sw.lora_a, "bf16", y, "f32", sw.start, sw.lens, sw.idx, 1.0)
    # |y| <= 9 * 20 = 180 < 256: bf16-exact, so the expand's cast keeps it
    rng = np.random.default_rng(22)
    b = W.integers_as(rng, (L, N, K), -1, 1, "bf16")
    out = np.zeros((sw.T, N), dtype=np.float32)
    oracle.expand([oracle.Slice(y[0], "f32", b, "bf16", 0)], out, "f32", sw.start, sw.lens,
                  sw.idx, False, K, L)
    x = np_values(sw.x, "bf16").astype(np.int64)
    av = np_values(sw.lora_a[0], "bf16").astype(np.int64)
    bv = np_values(b, "bf16").astype(np.int64)
    ra = row_adapters(sw)
    for t in range(sw.T):
        if ra[t] < 0:
            assert np.all(out[t] == 0)
            continue
        delta = x[t] @ av[ra[t]].T @ bv[ra[t]].T
        assert np.array_equal(out[t], delta.astype(np.float32)), t


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------

def test_scaling_is_linear():
    wl = W.shrink_custom([9, 5], [0, 1], H=48, K=16, L=2, out_dtype="f32", seed=5)
    _, r1 = run_shrink(wl, scale=1.0)
    _, r4 = run_shrink(wl, scale=4.0)
    _, r3 = run_shrink(wl, scale=0.3)
    assert np.array_equal(r4[0], 4.0 * r1[0])  # power of two: exact in fp64
    assert np.allclose(r3[0], 0.3 * r1[0], rtol=1e-15, atol=0)


def test_row_subset_matches_full_call():
    wl = W.shrink_custom([12, 9, 7], [1, -1, 0], H=64, K=8, L=2, slices=2, seed=6)
    full, rfull = run_shrink(wl)
    rows = np.array([0, 5, 11, 12, 20, 27], dtype=np.int64)
    part, rpart = run_shrink(wl, rows=rows)
    written = np.zeros(wl.T, dtype=bool)
    written[rows] = True
    for si in range(2):
        assert np.array_equal(part[si][rows], full[si][rows])
        assert np.array_equal(part[si][~written], wl.outs0[si][~written])
        ok = ~np.isnan(rpart[si][:, 0])
        # rows 12..20 form the index -1 segment
        assert np.array_equal(np.nonzero(ok)[0], [0, 5, 11, 27])


def test_multi_slice_equals_separate_calls():
    wl = W.shrink_custom([10, 3, 8], [0, 2, 1], H=40, K=16, L=3, slices=3, seed=7)
    together, _ = run_shrink(wl)
    for si in range(3):
        alone = wl.outs0[si].copy()
        oracle.shrink(wl.x, wl.x_dtype, [wl.lora_a[si]], wl.a_dtype, [alone], wl.out_dtype,
                      wl.start, wl.lens, wl.idx, wl.scale)
        assert np.array_equal(alone, together[si])


def test_threads_do_not_change_results():
    wl = W.shrink_custom([40, 25, 33], [0, 1, 0], H=96, K=24, L=2, seed=8)
    one, _ = run_shrink(wl, threads=1)
    many, _ = run_shrink(wl, threads=5)
    assert np.array_equal(one[0], many[0])


def test_strided_rows():
    wl = W.shrink_custom([6, 5], [1, 0], H=32, K=8, L=2, x_pad=8, out_pad=4, seed=9)
    outs, ref = run_shrink(wl)
    y = masked_projection(wl)
    assert np.allclose(ref[0], y, rtol=1e-12, atol=1e-13)
    assert_rounded_from(outs[0], y, "bf16")


def test_rejects_bad_arguments():
    wl = W.shrink_custom([4, 4], [0, 1], H=16, K=8, L=2, seed=10)
    with pytest.raises(oracle.OracleError) as e:   # index >= lora_num
        oracle.shrink(wl.x, "bf16", wl.lora_a, "bf16", [o.copy() for o in wl.outs0], "bf16",
                      wl.start, wl.lens, np.array([0, 2]), 1.0)
    assert e.value.code == oracle.BAD_INDEX
    with pytest.raises(oracle.OracleError) as e:   # overlapping segments
        oracle.shrink(wl.x, "bf16", wl.lora_a, "bf16", [o.copy() for o in wl.outs0], "bf16",
                      np.array([0, 2]), wl.lens, wl.idx, 1.0)
    assert e.value.code == oracle.BAD_SEGMENT
    with pytest.raises(oracle.OracleError) as e:   # fp16 input with bf16 weights
        x16 = np.zeros_like(wl.x)
        oracle.shrink(x16, "f16", wl.lora_a, "bf16", [o.copy() for o in wl.outs0], "bf16",
                      wl.start, wl.lens, wl.idx, 1.0)
    assert e.value.code == oracle.BAD_ARGUMENT
