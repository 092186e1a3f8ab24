"""Pins of the fused LoRA delta reference (oracle.fused: the shrink into the
weights' 16-bit dtype, then the expand).  Reading: the fused call computes
what the two calls compute with the projection stored in the weights'
dtype -- the expand's inputs have the weights' dtype (or float32, which the
expand rounds to that dtype anyway).  Pinned against numpy integer
arithmetic (a dense x . A^T . B^T), against hand-built cases where the
projection's rounding to bfloat16 decides the result, and by slice
independence."""
import numpy as np
import pytest

import oracle
import sgmv_workloads as W
from oracle_pins_util import np_values, row_adapters


def run_fused(wl, want_ref=False):
    out = wl.out0.copy()
    ys, ref = oracle.fused(wl.x, wl.x_dtype, wl.lora_a, wl.lora_b, wl.w_dtype, wl.offsets, out,
                           wl.out_dtype, wl.start, wl.lens, wl.idx, wl.scale, wl.add,
                           want_ref=want_ref)
    return out, ys, ref


@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("w_dtype,out_dtype,x_dtype", [("bf16", "f32", "bf16"),
                                                       ("f16", "f16", "f16"),
                                                       ("bf16", "f32", "f32")])
def test_integer_data_equals_dense_lora_delta(add, w_dtype, out_dtype, x_dtype):
    # |y| <= 16 * 2 * 2 = 64 is exact in bf16 and f16; |out| <= 8 + 8 * 64 * 2
    # = 1032 is exact in f16 and f32
    wl = W.fused_custom([5, 0, 9, 3, 7], [1, 0, -1, 2, 1], H=16, K=8, L=3,
                        slices=[(4, 24), (40, 16), (60, 8)], H_out=72, x_dtype=x_dtype,
                        w_dtype=w_dtype, out_dtype=out_dtype, add=add, values="int", seed=7)
    out, ys, _ = run_fused(wl)
    ra = row_adapters(wl)
    x = np_values(wl.x, wl.x_dtype).astype(np.int64)
    exp = np_values(wl.out0, wl.out_dtype).astype(np.int64)
    for a_s, b_s, off in zip(wl.lora_a, wl.lora_b, wl.offsets):
        av = np_values(a_s, w_dtype).astype(np.int64)
        bv = np_values(b_s, w_dtype).astype(np.int64)
        n = b_s.shape[1]
        for t in np.nonzero(ra >= 0)[0]:
            y = av[ra[t]] @ x[t]
            base = exp[t, off:off + n] if add else 0
            exp[t, off:off + n] = base + bv[ra[t]] @ y
    got = np_values(out, wl.out_dtype)
    assert np.array_equal(got, exp.astype(np.float64))
    # the projections handed to the expand are the exact integers
    for y, a_s in zip(ys, wl.lora_a):
        av = np_values(a_s, w_dtype).astype(np.int64)
        for t in np.nonzero(ra >= 0)[0]:
            assert np.array_equal(np_values(y[t:t + 1], w_dtype)[0], av[ra[t]] @ x[t])


def _one_value_case(x_row, a_row, scale):
    """T = 1, rank 1, hidden len(x_row), one slice of width 1 with lora_B =
    1: the output is the projection itself, rounded to bfloat16, in
    float32."""
    H = len(x_row)
    bf = lambda v: W._to_storage(np.asarray(v, dtype=np.float32), "bf16")
    x = bf([x_row])
    a = bf([[a_row]])                    # (L=1, K=1, H)
    b = bf([[[1.0]]])                    # (L=1, N=1, K=1)
    wl = W.FusedWorkload("one", x, "bf16", [a], [b], "bf16", [0], np.zeros((1, 1), np.float32),
                         "f32", np.array([0]), np.array([1]), np.array([0]), scale, False, 1, 1)
    out, ys, _ = run_fused(wl)
    return float(out[0, 0]), float(np_values(ys[0], "bf16")[0, 0])


def test_projection_rounds_to_bf16_before_the_expand():
    # 1 + 2^-9 is not a bfloat16 value (8 significant bits); it rounds to 1
    got, y = _one_value_case([1.0, 2.0 ** -9], [1.0, 1.0], 1.0)
    assert y == 1.0 and got == 1.0
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even, 1
    got, _ = _one_value_case([1.0, 2.0 ** -8], [1.0, 1.0], 1.0)
    assert got == 1.0
    # 1 + 3 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: ties to even, 1 + 2^-6
    got, _ = _one_value_case([1.0, 3 * 2.0 ** -8], [1.0, 1.0], 1.0)
    assert got == 1.0 + 2.0 ** -6
    # 1 + 2^-7 is representable and kept
    got, _ = _one_value_case([1.0, 2.0 ** -7], [1.0, 1.0], 1.0)
    assert got == 1.0 + 2.0 ** -7


def test_scale_applies_before_the_rounding():
    # scale 1/2 of 2 + 2^-8 is 1 + 2^-9, which rounds to 1 (not 1 + 2^-8 / 2
    # rounded after scaling the rounded 2)
    got, _ = _one_value_case([2.0, 2.0 ** -8], [1.0, 1.0], 0.5)
    assert got == 1.0
    # scale 3: 3 (1 + 2^-8) = 3 + 3 2^-8 rounds to 3 + 2^-6 (bf16 spacing 2^-6 at 3)
    got, _ = _one_value_case([1.0, 2.0 ** -8], [1.0, 1.0], 3.0)
    assert got == 3.0 + 2.0 ** -6


def test_slices_are_independent():
    wl = W.fused_custom([20, 3, 11], [0, 1, 0], H=64, K=16, L=2,
                        slices=[(0, 40), (48, 24), (80, 16)], H_out=96, add=True, seed=9)
    out, _, _ = run_fused(wl)
    one = wl.out0.copy()
    for i in range(3):
        oracle.fused(wl.x, wl.x_dtype, [wl.lora_a[i]], [wl.lora_b[i]], wl.w_dtype,
                     [wl.offsets[i]], one, wl.out_dtype, wl.start, wl.lens, wl.idx, wl.scale,
                     wl.add)
    assert np.array_equal(out, one)


def test_rows_without_adapter_and_other_columns_untouched():
    wl = W.fused_custom([6, 4, 5], [1, -1, 0], H=32, K=8, L=2, slices=[(8, 16)], H_out=40,
                        add=False, seed=11)
    out, _, _ = run_fused(wl)
    assert np.array_equal(out[6:10], wl.out0[6:10])
    assert np.array_equal(out[:, :8], wl.out0[:, :8])
    assert np.array_equal(out[:, 24:], wl.out0[:, 24:])
    assert not np.array_equal(out[:6, 8:24], wl.out0[:6, 8:24])
