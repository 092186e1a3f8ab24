"""Pins for the CPU oracle against facts fixed outside the oracle itself.

* the page's worked example (segment lengths [4, 6] start at rows [0, 4]);
* special cases that reduce to a plain matrix product (numpy BLAS);
* exact integer-valued cases, compared bit for bit with numpy integer math;
* brute force on tiny inputs through a differently structured reference
  (per-adapter row masks and numpy matrix products);
* the invariants of the operation (untouched regions bit-identical,
  independence of segment order and splitting, power-of-two scaling,
  idempotent overwrite, accumulate = prior + overwrite result);
* the float32-input cast against library conversions;
* the comparator catching planted mistakes.

Page: "Implementation: Predibase Lorax SGMV Expand Slice Kernel" (Description;
I/O Contract, Inputs and Outputs; Usage Examples).
"""
import json
import os

import numpy as np
import pytest

import oracle
import sgmv_workloads as W
from oracle_pins_util import masked_reference, np_values, row_adapters, ulp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run_oracle(wl, want_ref=True, threads=0):
    out = wl.out0.copy()
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]
    ref = oracle.expand(slices, out, wl.out_dtype, wl.start, wl.lens, wl.idx, wl.add,
                        wl.K, wl.L, want_ref=want_ref, threads=threads)
    return out, ref


def assert_matches_reference(wl, out, ref):
    """Oracle output vs the masked numpy reference: untouched bits identical,
    written values within half an ulp of the exact value, fp64 values within
    rounding noise."""
    expected, written = masked_reference(wl)
    assert np.array_equal(out[~written], wl.out0[~written]), "untouched region changed"
    got = np_values(out, wl.out_dtype)[written]
    exp = expected[written]
    err = np.abs(got - exp)
    assert np.all(err <= 0.5 * ulp(exp, wl.out_dtype) * (1 + 1e-9) + 1e-300), err.max()
    ra = row_adapters(wl)
    rows = ra >= 0
    for s, r in zip(wl.slices, ref):
        e = expected[:, s.offset:s.offset + s.N][rows]
        scale = 1.0 + np.abs(e)
        assert np.all(np.abs(r[rows] - e) <= 1e-12 * scale)
        assert np.all(np.isnan(r[~rows]))


# --------------------------------------------------------------------------
# Worked example and usage example printed on the page.
# --------------------------------------------------------------------------

def test_worked_example_starts():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    assert W.exclusive_cumsum(g["seq_lens"]).tolist() == g["b_seq_start_loc"]
    wl = W.tiny_ref(0)
    assert wl.lens.tolist() == g["seq_lens"]
    assert wl.start.tolist() == g["b_seq_start_loc"]
    assert wl.T == g["total_tokens"]


def test_worked_example_rows_follow_segments():
    """With lengths [4, 6] at starts [0, 4], adapter 1 on the first segment and
    adapter 0 on the second, rows 0-3 use adapter 1 and rows 4-9 adapter 0."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    wl = W.custom(g["seq_lens"], [1, 0], K=8, N=64, H=192, off=64, L=2, x_dtype="f16",
                  w_dtype="f16", out_dtype="f32", start=g["b_seq_start_loc"], seed=5)
    out, ref = run_oracle(wl)
    xv = np_values(wl.slices[0].x, "f16")
    wv = np_values(wl.slices[0].w, "f16")
    assert np.allclose(ref[0][0:4], xv[0:4] @ wv[1].T, rtol=1e-12, atol=1e-14)
    assert np.allclose(ref[0][4:10], xv[4:10] @ wv[0].T, rtol=1e-12, atol=1e-14)
    assert_matches_reference(wl, out, ref)


def test_tiny_ref_index_minus_one_rows_untouched():
    wl = W.tiny_ref(0)
    out, ref = run_oracle(wl)
    assert np.array_equal(out[4:], wl.out0[4:])            # idx -1 segment
    assert np.array_equal(out[:, :64], wl.out0[:, :64])    # left of the slice
    assert np.array_equal(out[:, 128:], wl.out0[:, 128:])  # right of the slice
    assert not np.array_equal(out[:4, 64:128], wl.out0[:4, 64:128])
    assert_matches_reference(wl, out, ref)


def test_usage_example_q_slice():
    """Query window of a fused QKV output, offset 0, accumulate (Usage Examples)."""
    g = json.load(open(os.path.join(GOLDEN, "usage_qkv_q_slice.json")))
    wl = W.custom([3, 5, 2], [0, 1, 0], K=16, N=128, H=3 * 128, off=g["slice_offset"], L=2,
                  add=g["add_inputs"], seed=6)
    assert wl.slices[0].w.shape[1] == wl.slices[0].N   # slice_size == lora_b rows
    out, ref = run_oracle(wl)
    assert np.array_equal(out[:, 128:], wl.out0[:, 128:])
    assert_matches_reference(wl, out, ref)


# --------------------------------------------------------------------------
# Special cases that reduce to a plain matrix product.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("out_dtype", ["f32", "f16", "bf16"])
def test_single_segment_is_a_gemm(out_dtype):
    """One segment over every row, adapter 0, slice = whole row, overwrite:
    out = rne(X @ W0^T).  N != K so a transposed operand cannot pass."""
    T, K, N = 37, 24, 40
    wl = W.custom([T], [0], K=K, N=N, H=N, off=0, L=3, out_dtype=out_dtype, seed=7)
    out, ref = run_oracle(wl)
    gemm = np_values(wl.slices[0].x, "bf16") @ np_values(wl.slices[0].w, "bf16")[0].T
    assert np.allclose(ref[0], gemm, rtol=1e-12, atol=1e-13)
    got = np_values(out, out_dtype)
    assert np.all(np.abs(got - gemm) <= 0.5 * ulp(gemm, out_dtype) * (1 + 1e-9))


def test_shared_adapter_is_one_gemm_over_concatenated_rows():
    wl = W.custom([5, 9, 3, 7], [2, 2, 2, 2], K=16, N=48, H=64, off=8, L=3,
                  out_dtype="f32", seed=8)
    out, ref = run_oracle(wl)
    gemm = np_values(wl.slices[0].x, "bf16") @ np_values(wl.slices[0].w, "bf16")[2].T
    assert np.allclose(ref[0], gemm, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Exact integer-valued cases: every product and partial sum is an exact small
# integer (|r| <= 8 + 16*9 = 152 < 256), so the result is known bit for bit.
# --------------------------------------------------------------------------

def _int_expected_bits(wl):
    ra = row_adapters(wl)
    expected = wl.out0.copy()
    prior_int = np_values(wl.out0, wl.out_dtype).astype(np.int64)
    for s in wl.slices:
        x = np_values(np.ascontiguousarray(s.x), s.x_dtype).astype(np.int64)
        w = np_values(s.w, s.w_dtype).astype(np.int64)
        for t in range(wl.T):
            a = ra[t]
            if a < 0:
                continue
            r = x[t] @ w[a].T
            if wl.add:
                r = r + prior_int[t, s.offset:s.offset + s.N]
            rf = r.astype(np.float32)
            if wl.out_dtype == "f32":
                bits = rf
            elif wl.out_dtype == "f16":
                bits = rf.astype(np.float16).view(np.uint16)
            else:
                bits = (rf.view(np.uint32) >> 16).astype(np.uint16)   # exact: |r| < 256
            expected[t, s.offset:s.offset + s.N] = bits
    return expected


@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("x_dtype,w_dtype,out_dtype", [
    ("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("f32", "bf16", "bf16"),
    ("f32", "f16", "f32"), ("bf16", "bf16", "f32"), ("f16", "f16", "bf16")])
def test_integer_cases_exact(add, x_dtype, w_dtype, out_dtype):
    wl = W.custom([3, 0, 6, 4, 5], [1, 0, -1, 0, 2], K=13, N=21, H=40, off=11, L=3,
                  x_dtype=x_dtype, w_dtype=w_dtype, out_dtype=out_dtype, add=add,
                  values="int", seed=9)
    out, _ = run_oracle(wl)
    assert np.array_equal(out, _int_expected_bits(wl))


# --------------------------------------------------------------------------
# Brute force on tiny random inputs through the masked reference.
# --------------------------------------------------------------------------

def _tiny_cases():
    rng = np.random.default_rng(10)
    cases = []
    dts = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("f32", "bf16", "bf16"),
           ("f32", "f16", "f16"), ("bf16", "bf16", "f32"), ("f16", "f16", "f32")]
    for i in range(40):
        B = int(rng.integers(0, 5))
        L = int(rng.integers(1, 4))
        lens = rng.integers(0, 5, size=B)
        idx = rng.integers(-1, L, size=B)
        K = int(rng.integers(1, 18))
        N = int(rng.integers(1, 21))
        H = N + int(rng.integers(0, 9))
        off = int(rng.integers(0, H - N + 1))
        cases.append(dict(lens=lens.tolist(), idx=idx.tolist(), K=K, N=N, H=H, off=off, L=L,
                          dt=dts[i % len(dts)], add=bool(i % 2), seed=100 + i))
    return cases


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: f"B{len(c['lens'])}K{c['K']}N{c['N']}")
def test_brute_force_tiny(case):
    x_dt, w_dt, o_dt = case["dt"]
    # permuted starts with a gap row in front: segment order != row order
    lens = case["lens"]
    order = np.random.default_rng(case["seed"]).permutation(len(lens))
    start = np.zeros(len(lens), dtype=np.int64)
    pos = 1
    for b in order:
        start[b] = pos
        pos += lens[b]
    wl = W.custom(lens, case["idx"], K=case["K"], N=case["N"], H=case["H"], off=case["off"],
                  L=case["L"], x_dtype=x_dt, w_dtype=w_dt, out_dtype=o_dt, add=case["add"],
                  seed=case["seed"], start=start, T=pos + 1)
    out, ref = run_oracle(wl)
    assert_matches_reference(wl, out, ref)


def test_brute_force_multi_slice():
    wl = W.custom([4, 3, 5], [1, -1, 0], K=9, N=10, H=40, off=3, L=2, add=True, seed=11,
                  extra_slices=[(20, 7), (13, 5)])
    out, ref = run_oracle(wl)
    assert_matches_reference(wl, out, ref)


# --------------------------------------------------------------------------
# The per-token (BGMV) form.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,add,dts", [(31, False, ("bf16", "bf16", "bf16")),
                                          (32, True, ("f16", "f16", "f32")),
                                          (33, True, ("f32", "bf16", "f16"))])
def test_bgmv_per_token_brute_force(seed, add, dts):
    # Every row takes its own adapter; checked through the masked reference,
    # which reads the per-row adapters from (start t, length 1) segments.
    x_dt, w_dt, o_dt = dts
    idx = np.random.default_rng(seed).integers(-1, 4, size=23)
    wl = W.per_token(idx.tolist(), K=11, N=13, H=30, off=9, L=4, x_dtype=x_dt, w_dtype=w_dt,
                     out_dtype=o_dt, add=add, seed=seed)
    out = wl.out0.copy()
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]
    ref = oracle.bgmv_expand(slices, out, wl.out_dtype, wl.idx, wl.add, wl.K, wl.L,
                             want_ref=True)
    assert_matches_reference(wl, out, ref)


def test_bgmv_row_by_row_matrix_vector():
    # Token t's slice equals x[t] @ W[idx[t]]^T computed on its own (a plain
    # matrix-vector product per row), exactly for integer values.
    idx = [2, 0, -1, 2, 1, 0]
    wl = W.per_token(idx, K=5, N=7, H=7, off=0, L=3, x_dtype="f16", w_dtype="f16",
                     out_dtype="f32", values="int", seed=34)
    out = wl.out0.copy()
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]
    oracle.bgmv_expand(slices, out, "f32", wl.idx, False, wl.K, wl.L)
    x = np_values(wl.slices[0].x, "f16").astype(np.int64)
    w = np_values(wl.slices[0].w, "f16").astype(np.int64)
    for t, a in enumerate(idx):
        if a < 0:
            assert np.array_equal(out[t], wl.out0[t])
        else:
            assert np.array_equal(out[t].astype(np.int64), w[a] @ x[t])


# --------------------------------------------------------------------------
# Invariants.
# --------------------------------------------------------------------------

def test_segment_order_does_not_matter():
    wl = W.custom([5, 3, 7, 2], [0, 2, -1, 1], K=16, N=24, H=32, off=4, L=3, add=True, seed=12)
    out1, _ = run_oracle(wl)
    p = np.array([2, 0, 3, 1])
    wl.start, wl.lens, wl.idx = wl.start[p], wl.lens[p], wl.idx[p]
    out2, _ = run_oracle(wl)
    assert np.array_equal(out1, out2)


def test_splitting_a_segment_changes_nothing():
    wl = W.custom([9], [1], K=8, N=16, H=16, off=0, L=2, seed=13)
    out1, _ = run_oracle(wl)
    wl.start, wl.lens, wl.idx = np.array([0, 4]), np.array([4, 5]), np.array([1, 1])
    out2, _ = run_oracle(wl)
    assert np.array_equal(out1, out2)


def test_power_of_two_scaling():
    wl = W.custom([6, 4], [0, 1], K=12, N=20, H=20, off=0, L=2, out_dtype="f32", seed=14)
    out1, _ = run_oracle(wl)
    w = wl.slices[0].w
    wl.slices[0].w = (w.astype(np.uint32) + (1 << 7)).astype(np.uint16)  # bf16 exponent + 1
    out2, _ = run_oracle(wl)
    assert np.array_equal(out2.astype(np.float64), 2.0 * out1.astype(np.float64))


def test_overwrite_is_idempotent():
    wl = W.custom([6, 4], [0, 1], K=12, N=20, H=24, off=2, L=2, seed=15)
    out1, _ = run_oracle(wl)
    wl.out0 = out1.copy()
    out2, _ = run_oracle(wl)
    assert np.array_equal(out1, out2)


def test_accumulate_equals_prior_plus_overwrite():
    wl = W.custom([6, 4, 3], [0, 1, -1], K=12, N=20, H=24, off=2, L=2, seed=16)
    wl.add = False
    _, ref0 = run_oracle(wl)
    wl.add = True
    _, ref1 = run_oracle(wl)
    prior = np_values(wl.out0, "bf16")[:, 2:22]
    rows = row_adapters(wl) >= 0
    assert np.allclose(ref1[0][rows], prior[rows] + ref0[0][rows], rtol=1e-13, atol=1e-14)


def test_float32_input_is_cast_to_weight_dtype():
    """float32 inputs holding bf16-exact values give the bf16-input result;
    arbitrary float32 inputs give the result of the inputs rounded by torch."""
    import torch
    wl = W.custom([5, 6], [1, 0], K=16, N=24, H=24, off=0, L=2, x_dtype="f32",
                  w_dtype="bf16", out_dtype="f32", seed=17)
    out_f32, _ = run_oracle(wl)
    rounded = torch.from_numpy(wl.slices[0].x).to(torch.bfloat16)
    wl.slices[0].x = rounded.view(torch.int16).numpy().view(np.uint16).copy()
    wl.slices[0].x_dtype = "bf16"
    out_bf16, _ = run_oracle(wl)
    assert np.array_equal(out_f32, out_bf16)


# --------------------------------------------------------------------------
# Error handling and the comparator.
# --------------------------------------------------------------------------

def test_rejects_bad_segments_and_indices():
    wl = W.custom([3, 4], [0, 1], K=8, N=8, H=8, off=0, L=2, seed=18)
    base = dict(slices=[oracle.Slice(wl.slices[0].x, "bf16", wl.slices[0].w, "bf16", 0)],
                out_dtype="bf16", add_inputs=False, K=8, L=2)
    for start, lens, idx, code in [
        ([0, 3], [3, 4], [0, 2], oracle.BAD_INDEX),
        ([0, 3], [3, 4], [-2, 0], oracle.BAD_INDEX),
        ([0, 4], [3, 4], [0, 1], oracle.BAD_SEGMENT),     # runs past T
        ([0, 2], [3, 4], [0, 1], oracle.BAD_SEGMENT),     # overlap
        ([-1, 3], [3, 4], [0, 1], oracle.BAD_SEGMENT),
    ]:
        out = wl.out0.copy()
        with pytest.raises(oracle.OracleError) as e:
            oracle.expand(out=out, start=start, lens=lens, idx=idx, **base)
        assert e.value.code == code
        assert np.array_equal(out, wl.out0)
    # overlap with an index -1 segment is fine: it writes nothing
    out = wl.out0.copy()
    oracle.expand(out=out, start=[0, 2], lens=[3, 4], idx=[0, -1], **base)


def test_rejects_bad_slices():
    wl = W.custom([3], [0], K=8, N=8, H=16, off=0, L=1, seed=19)
    s = wl.slices[0]
    for slices in ([oracle.Slice(s.x, "bf16", s.w, "bf16", 9)],                 # past H
                   [oracle.Slice(s.x, "bf16", s.w, "bf16", 0),
                    oracle.Slice(s.x, "bf16", s.w, "bf16", 4)],                 # overlap
                   [oracle.Slice(s.x.view(np.uint16), "f16", s.w, "bf16", 0)]):  # mixed 16-bit
        with pytest.raises(oracle.OracleError):
            oracle.expand(slices, wl.out0.copy(), "bf16", wl.start, wl.lens, wl.idx, False, 8, 1)


def test_comparator_catches_planted_mistakes():
    wl = W.custom([5, 4, 3], [0, -1, 1], K=16, N=24, H=40, off=8, L=2, add=True, seed=20)
    out, _ = run_oracle(wl)
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]
    args = (slices, wl.out0, None, "bf16", wl.start, wl.lens, wl.idx, True, 16, 2, 1e-3, 8e-3)

    def chk(cand):
        a = list(args)
        a[2] = cand
        return oracle.check(*a)

    rep = chk(out)
    assert rep.ok and rep.checked_values == 8 * 24 and rep.checked_untouched == 12 * 40 - 8 * 24
    bad = out.copy()
    v = np_values(bad[2:3, 10:11], "bf16")[0, 0]
    bad[2, 10] = (np.array([v * 1.1 + 0.05], dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)[0]
    rep = chk(bad)
    assert rep.bad_values == 1 and rep.first_bad == (2, 10)
    bad = out.copy()
    bad[6, 12] ^= 1                     # a row of the index -1 segment
    rep = chk(bad)
    assert rep.bad_untouched == 1 and rep.first_bad == (6, 12)
    bad = out.copy()
    bad[0, 39] ^= 1                     # right of the slice
    assert chk(bad).bad_untouched == 1
    bad = out.copy()
    bad[1, 8] = 0x7FC0                  # NaN where a finite value belongs
    assert chk(bad).bad_values == 1
    rows = np.array([0, 6])
    rep = oracle.check(slices, wl.out0, out, "bf16", wl.start, wl.lens, wl.idx, True, 16, 2,
                       1e-3, 8e-3, rows=rows)
    assert rep.ok and rep.checked_values == 24 and rep.checked_untouched == 2 * 40 - 24


def test_threads_do_not_change_results():
    wl = W.custom([50, 70, 30], [0, 1, 0], K=16, N=64, H=64, off=0, L=2, add=True, seed=21)
    out1, _ = run_oracle(wl, threads=1)
    out4, _ = run_oracle(wl, threads=4)
    assert np.array_equal(out1, out4)
