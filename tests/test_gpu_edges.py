"""GPU edge-case parity: ranks and slice widths around every tile boundary,
ragged tails, misaligned offsets and strides, empty and degenerate segment
layouts, exact integer cases, the float32 cast, epilogue rounding, NaN
containment, multi-slice identity, wrapper forms and device-side guard
bands.  Every result is compared with the CPU oracle (or, where the claim is
bit-identity between two GPU calls, with the other call)."""
import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceWorkload, assert_parity, to_device, to_host_bits

pytestmark = pytest.mark.gpu

DTYPES = [("bf16", "bf16", "bf16"), ("f16", "f16", "f16"), ("f32", "bf16", "bf16"),
          ("f32", "f16", "f32"), ("bf16", "bf16", "f32"), ("f16", "f16", "bf16")]


def run_and_check(wl, multi=False):
    dw = DeviceWorkload(wl)
    out = dw.fresh_out()
    out = dw.run_multi(out) if multi else dw.run_all_single(out)
    bits = to_host_bits(out)
    assert_parity(wl, bits)
    return dw, bits


@pytest.mark.parametrize("K", [1, 7, 8, 15, 16, 17, 31, 32, 33, 48, 64, 65, 100, 127, 128, 129,
                               200, 255, 256])
def test_rank_sweep(K):
    x, w, o = DTYPES[K % len(DTYPES)]
    wl = W.custom([17, 0, 33, 5, 40], [1, 0, -1, 2, 1], K=K, N=300, H=320, off=8, L=3,
                  x_dtype=x, w_dtype=w, out_dtype=o, add=bool(K % 2), seed=K)
    run_and_check(wl)


@pytest.mark.parametrize("N", [1, 7, 8, 9, 63, 64, 65, 255, 256, 257, 520, 4097])
def test_slice_width_sweep(N):
    x, w, o = DTYPES[N % len(DTYPES)]
    wl = W.custom([16, 3, 21], [0, 1, 0], K=16, N=N, H=N + 24, off=16, L=2,
                  x_dtype=x, w_dtype=w, out_dtype=o, add=bool(N % 2), seed=N)
    run_and_check(wl)


@pytest.mark.parametrize("off", [0, 1, 3, 7, 8, 9, 15, 33])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_misaligned_offsets(off, out_dtype):
    wl = W.custom([20, 9], [1, 0], K=32, N=130, H=200, off=off, L=2, out_dtype=out_dtype,
                  add=True, seed=off)
    run_and_check(wl)


@pytest.mark.parametrize("x_pad,out_pad", [(1, 0), (0, 3), (5, 7), (8, 8), (24, 16)])
def test_strided_inputs_and_output(x_pad, out_pad):
    wl = W.custom([13, 30], [0, 1], K=24, N=96, H=112, off=8, L=2, add=True, seed=40 + x_pad,
                  x_pad=x_pad, out_pad=out_pad)
    dw, bits = run_and_check(wl)
    # the padding columns of a strided output are never touched
    out = dw.run_single(dw.fresh_out())
    assert out.stride(0) == wl.H + out_pad
    full = out.as_strided((wl.T, wl.H + out_pad), (wl.H + out_pad, 1))
    if out_pad:
        assert (full[:, wl.H:] == 0).all()
    # same result as contiguous copies of the same values
    wl2 = W.Workload(wl.name, [W.SliceInput(np.ascontiguousarray(s.x), s.x_dtype, s.w, s.w_dtype,
                                            s.offset) for s in wl.slices],
                     np.ascontiguousarray(wl.out0), wl.out_dtype, wl.start, wl.lens, wl.idx,
                     wl.add, wl.K, wl.L)
    dw2 = DeviceWorkload(wl2)
    assert np.array_equal(to_host_bits(dw2.run_single(dw2.fresh_out())), bits)


LAYOUTS = {
    "zero_length": dict(lens=[0, 5, 0, 0, 7, 0], idx=[0, 1, 1, 0, 0, 1]),
    "all_minus_one": dict(lens=[5, 7, 3], idx=[-1, -1, -1]),
    "one_segment_gemm": dict(lens=[77], idx=[1]),
    "repeated_adapter": dict(lens=[9, 4, 16, 1, 33], idx=[1, 1, 1, 1, 1]),
    "many_tiny": dict(lens=[1] * 40 + [2] * 20, idx=[i % 3 - 1 for i in range(60)]),
}


@pytest.mark.parametrize("name", sorted(LAYOUTS))
@pytest.mark.parametrize("add", [False, True])
def test_segment_layouts(name, add):
    lay = LAYOUTS[name]
    wl = W.custom(lay["lens"], lay["idx"], K=16, N=256, H=272, off=16, L=2, add=add,
                  seed=len(lay["lens"]))
    dw, bits = run_and_check(wl)
    if name == "all_minus_one":
        assert np.array_equal(bits, wl.out0)


def test_gaps_and_unsorted_starts():
    lens = [6, 17, 3, 40, 2]
    start = [90, 3, 60, 20, 70]          # any order, gaps between segments
    wl = W.custom(lens, [1, 0, 2, 1, -1], K=32, N=200, H=240, off=24, L=3, add=True, seed=3,
                  start=start, T=100)
    run_and_check(wl)


def test_many_segments_multi_chunk_scan():
    rng = np.random.default_rng(4)
    B = 3900
    lens = rng.integers(0, 4, size=B)
    idx = rng.integers(-1, 6, size=B)
    wl = W.custom(lens.tolist(), idx.tolist(), K=16, N=64, H=64, off=0, L=6, seed=4)
    run_and_check(wl)



@pytest.mark.parametrize("B", [1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 100])
def test_segment_counts_around_the_wave_scan(B):
    # Up to 64 segments the row-tile prefix sums are taken in one wave's
    # registers (a scan inside 16-lane rows, then across the rows); more
    # segments take the workgroup-wide path.  Inactive segments in between.
    rng = np.random.default_rng(500 + B)
    lens = rng.integers(1, 40, size=B)
    idx = rng.integers(-1, 5, size=B)
    wl = W.custom(lens.tolist(), idx.tolist(), K=16, N=256, H=256, off=0, L=5, add=True,
                  seed=B)
    run_and_check(wl)

def shuffled_placement(rng, lens):
    """Start rows for segments placed in a random order with small gaps."""
    start = np.zeros(len(lens), dtype=np.int64)
    row = 0
    for b in rng.permutation(len(lens)):
        row += int(rng.integers(0, 3))
        start[b] = row
        row += int(lens[b])
    return start, row


@pytest.mark.parametrize("B", [127, 128, 300, 512, 513])
def test_adapter_ordered_segment_table(B):
    # Batches of 128..512 segments get a segment table ordered by adapter
    # (neighbours share weight tiles); the result must not depend on it.
    rng = np.random.default_rng(100 + B)
    lens = rng.integers(0, 20, size=B)
    idx = rng.integers(-1, 12, size=B)
    start, T = shuffled_placement(rng, lens)
    wl = W.custom(lens.tolist(), idx.tolist(), K=64, N=512, H=576, off=32, L=12, add=True,
                  seed=B, start=start.tolist(), T=T)
    run_and_check(wl)



@pytest.mark.parametrize("B,L", [(128, 1023), (300, 1500), (512, 1100)])
def test_adapter_ordered_segment_table_many_adapters(B, L):
    # Adapter-ordered tables with up to 1500 adapters (the order is taken by
    # ranking (adapter, index) keys) and one crowded adapter.
    rng = np.random.default_rng(200 + B)
    lens = rng.integers(0, 12, size=B)
    idx = rng.integers(-1, L, size=B)
    idx[: B // 8] = L - 1  # a crowded last adapter
    start, T = shuffled_placement(rng, lens)
    wl = W.custom(lens.tolist(), idx.tolist(), K=16, N=64, H=64, off=0, L=L, add=True,
                  seed=B, start=start.tolist(), T=T)
    run_and_check(wl)

def test_strided_chunks_several_per_workgroup():
    # Enough 16x256 units that every workgroup takes several strided chunks
    # of its column group's walk; with 4 column tiles, half of the 8 column
    # groups are empty and their workgroups do nothing.
    rng = np.random.default_rng(7)
    lens = rng.integers(2000, 9000, size=16)
    idx = rng.integers(-1, 4, size=16)
    wl = W.custom(lens.tolist(), idx.tolist(), K=8, N=1024, H=1024, off=0, L=4, add=True,
                  out_dtype="f16", x_dtype="f16", w_dtype="f16", seed=7)
    assert wl.T >= 90000
    run_and_check(wl)



@pytest.mark.parametrize("dts", DTYPES)
def test_rank16_pipeline_several_units_and_adapter_changes(dts):
    # Rank <= 16 on contiguous rows keeps two units of loads in flight; here
    # workgroups hold several units each and the adapter (so the weight tile)
    # changes inside their chunks.
    rng = np.random.default_rng(77)
    B = 180
    lens = rng.integers(100, 300, size=B)
    idx = rng.integers(-1, 6, size=B)
    x, w, o = dts
    wl = W.custom(lens.tolist(), idx.tolist(), K=16, N=512, H=544, off=16, L=6,
                  x_dtype=x, w_dtype=w, out_dtype=o, add=True, seed=77)
    assert wl.T > 30000
    run_and_check(wl)

@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("dts", DTYPES)
def test_integer_cases_bit_exact(add, dts):
    """Small integers: every product and sum is exact, so the GPU result must
    equal the oracle's bit for bit."""
    import oracle
    x, w, o = dts
    wl = W.custom([3, 16, 6, 20, 5], [1, 0, -1, 0, 2], K=16, N=70, H=96, off=13, L=3,
                  x_dtype=x, w_dtype=w, out_dtype=o, add=add, values="int", seed=9)
    dw = DeviceWorkload(wl)
    bits = to_host_bits(dw.run_single(dw.fresh_out()))
    expect = wl.out0.copy()
    oracle.expand([oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices],
                  expect, o, wl.start, wl.lens, wl.idx, add, wl.K, wl.L)
    assert np.array_equal(bits, expect)


@pytest.mark.parametrize("w_dtype", ["bf16", "f16"])
def test_float32_input_cast_is_round_to_nearest_even(w_dtype):
    """float32 inputs are rounded to the weight dtype before the products: the
    result equals (bit for bit) the result for inputs rounded on the host by
    torch (round to nearest even)."""
    import torch
    wl = W.custom([11, 25, 7], [1, 0, 1], K=64, N=192, H=192, off=0, L=2, x_dtype="f32",
                  w_dtype=w_dtype, out_dtype="f32", add=True, seed=12)
    dw = DeviceWorkload(wl)
    got = to_host_bits(dw.run_single(dw.fresh_out()))
    tdt = torch.bfloat16 if w_dtype == "bf16" else torch.float16
    pre = torch.from_numpy(wl.slices[0].x).to(tdt).view(torch.int16).numpy().view(np.uint16)
    wl2 = W.Workload(wl.name, [W.SliceInput(pre, w_dtype, wl.slices[0].w, w_dtype, 0)],
                     wl.out0, "f32", wl.start, wl.lens, wl.idx, True, wl.K, wl.L)
    dw2 = DeviceWorkload(wl2)
    assert np.array_equal(to_host_bits(dw2.run_single(dw2.fresh_out())), got)
    assert_parity(wl, got)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("add", [False, True])
def test_epilogue_rounds_once_to_nearest_even(dt, add):
    """With rank 2, x = [1, 1] and prior, w chosen so that the fp32 sum is
    exact, the output is that sum rounded once to nearest even (ties
    included); expected bits come from numpy / torch conversions."""
    import torch
    rng = np.random.default_rng(13)
    T, N = 16, 256
    wl = W.custom([T], [0], K=2, N=N, H=N, off=0, L=1, x_dtype=dt, w_dtype=dt, out_dtype=dt,
                  add=add, seed=13)
    one = np.float32(1.0)
    x = np.full((T, 2), one, dtype=np.float32)
    # w0 in [1, 2) on the 16-bit grid, w1 = a multiple of 2^-12 below 2^-4:
    # w0 + w1 needs more significand bits than the output dtype has, often
    # landing exactly on a tie; the sum (and + prior) is exact in fp32.
    w0 = 1.0 + rng.integers(0, 8, size=N) / 8.0
    w1 = rng.integers(-256, 256, size=N) / 4096.0
    prior = (rng.integers(-8, 9, size=(T, N)) / 4.0) if add else np.zeros((T, N))
    wv = np.stack([w0, w1], axis=1)[None].astype(np.float32)
    if dt == "f16":
        enc = lambda a: a.astype(np.float16).view(np.uint16)
    else:
        enc = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for arr in (w0, w1):
        assert np.array_equal(arr.astype(np.float32), arr)  # representable as float32
    wl.slices[0].x = enc(x)
    wl.slices[0].w = enc(wv)
    wl.out0 = enc(prior.astype(np.float32))
    dw = DeviceWorkload(wl)
    got = to_host_bits(dw.run_single(dw.fresh_out()))
    # exact fp32 sum of representable values, rounded once by a library
    from oracle_pins_util import np_values
    exact = np.broadcast_to(np_values(wl.slices[0].w, dt)[0].sum(axis=1)[None, :], (T, N)) + \
        (np_values(wl.out0, dt) if add else 0.0)
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    assert np.array_equal(got, enc(exact.astype(np.float32)))


def test_nan_in_skipped_rows_and_unused_adapters_does_not_leak():
    wl = W.custom([6, 5, 7], [0, -1, 0], K=16, N=64, H=64, off=0, L=3, add=True, seed=14)
    x = wl.slices[0].x.copy()
    x[6:11] = 0x7FC0                       # NaN inputs in the index -1 segment
    w = wl.slices[0].w.copy()
    w[2] = 0x7FC0                          # NaN weights in an adapter nobody uses
    wl.slices[0].x, wl.slices[0].w = x, w
    dw, bits = run_and_check(wl)
    assert np.array_equal(bits[6:11], wl.out0[6:11])


@pytest.mark.parametrize("off", [8, 3])                # fast kernel; generic (misaligned)
@pytest.mark.parametrize("add", [False, True])
@pytest.mark.parametrize("dts", [("f16", "f16", "f16"), ("f32", "f16", "f32"),
                                 ("bf16", "bf16", "bf16"), ("f32", "bf16", "bf16")])
def test_nan_and_inf_in_active_rows_propagate(dts, add, off):
    """NaN and +-Inf in inputs, weights and prior output of active rows, an
    input cast that overflows, and sums that overflow f16 (see
    sgmv_workloads.nonfinite): every written element must be NaN exactly
    where the oracle's exact value is NaN, the same infinity where it rounds
    to one, within tolerance elsewhere; the index -1 segment's rows (with
    their own NaNs) keep their bits.  The data are integers, so every finite
    fp32 partial sum is exact."""
    wl = W.nonfinite(*dts, add=add, off=off)
    dw, bits = run_and_check(wl)
    from oracle_pins_util import np_values
    got = np_values(np.ascontiguousarray(bits[:, off:off + 64]), wl.out_dtype)
    assert np.isnan(got[1]).all() and np.isnan(got[6:11, 5]).all()
    assert np.isposinf(got[2]).any() and np.isneginf(got[2]).any()
    if add:
        assert np.isneginf(got[4, 5]) and np.isnan(got[5, 7])
    bview = bits.view(np.uint32) if wl.out_dtype == "f32" else bits
    oview = wl.out0.view(np.uint32) if wl.out_dtype == "f32" else wl.out0
    assert np.array_equal(bview[11:15], oview[11:15])


@pytest.mark.parametrize("add", [False, True])
def test_multi_slice_bit_identical_to_single_calls(add):
    # QKV-like three slices and gate/up-like two slices, ragged widths
    for extra, base in (([(300, 70), (370, 70)], (0, 300)), ([(256, 256)], (0, 256))):
        wl = W.custom([40, 3, 0, 19], [1, 0, 1, -1], K=32, N=base[1], H=512, off=base[0], L=2,
                      add=add, seed=15, extra_slices=extra)
        dw = DeviceWorkload(wl)
        single = to_host_bits(dw.run_all_single(dw.fresh_out()))
        fused = to_host_bits(dw.run_multi(dw.fresh_out()))
        assert np.array_equal(single, fused)
        assert_parity(wl, fused)


def test_wrapper_forms_give_identical_results():
    """4-D (L, 1, N, K) weights, int32 metadata and a loose max_seq_length
    give exactly the result of the plain call."""
    import torch
    import segmented_gather_gemm_amd as sg
    wl = W.custom([10, 20, 5], [1, 0, 1], K=16, N=128, H=160, off=16, L=2, add=True, seed=16)
    dw = DeviceWorkload(wl)
    ref = to_host_bits(dw.run_single(dw.fresh_out()))
    out = dw.fresh_out()
    sg.sgmv_expand_slice(dw.x[0], dw.w[0].unsqueeze(1), out, dw.start.int(), dw.lens.int(),
                         dw.idx.int(), wl.batches, 4096, 16, 128, True)
    assert np.array_equal(to_host_bits(out), ref)
    out = dw.run_single(dw.fresh_out(), max_seq_length=0)   # the hint is not needed
    assert np.array_equal(to_host_bits(out), ref)


def test_device_side_invalid_segments_are_skipped_inside_guard_bands():
    """Segments running past T, with a negative start or an index >= lora_num
    are skipped; nothing outside the output view is touched."""
    import torch
    import segmented_gather_gemm_amd as sg
    T, H, N, off = 40, 96, 64, 8
    good = W.custom([10, 12], [1, 0], K=16, N=N, H=H, off=off, L=2, add=True, seed=17, T=T)
    dw = DeviceWorkload(good)
    for pad_c, pad_r in ((1, 2), (8, 3)):          # misaligned and aligned views
        big = torch.full((T + 2 * pad_r, H + 2 * pad_c), 7.0, dtype=torch.bfloat16,
                         device="cuda")
        view = big[pad_r:pad_r + T, pad_c:pad_c + H]
        view.copy_(dw.out0)
        canary = big.clone()
        start = torch.tensor([0, 10, 30, -4, 35, 22], dtype=torch.int64, device="cuda")
        lens = torch.tensor([10, 12, 20, 6, 5, 3], dtype=torch.int64, device="cuda")
        idx = torch.tensor([1, 0, 1, 0, 2, 5], dtype=torch.int64, device="cuda")
        sg.sgmv_expand_slice(dw.x[0], dw.w[0], view, start, lens, idx, 6, 20, off, N, True)
        torch.cuda.synchronize()
        inner = torch.zeros_like(big, dtype=torch.bool)
        inner[pad_r:pad_r + T, pad_c:pad_c + H] = True
        assert torch.equal(big.view(torch.int16)[~inner], canary.view(torch.int16)[~inner])
        assert_parity(good, to_host_bits(view))


def test_empty_and_noop_calls_touch_nothing():
    import torch
    import segmented_gather_gemm_amd as sg
    wl = W.custom([0, 0, 0], [0, 1, 0], K=16, N=64, H=64, off=0, L=2, seed=18, T=8)
    dw = DeviceWorkload(wl)
    out = dw.run_single(dw.fresh_out())
    assert np.array_equal(to_host_bits(out), wl.out0)
    out = dw.fresh_out()
    sg.sgmv_expand_slice(dw.x[0], dw.w[0], out, dw.start, dw.lens, dw.idx, 0, 0, 0, 64, False)
    assert np.array_equal(to_host_bits(out), wl.out0)
