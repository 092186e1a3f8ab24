"""GPU parity of the fused LoRA delta (sgmv_fused_shrink_expand): the LoRA-A
projection and the expand of its result in one launch, against oracle.fused
(the oracle's shrink into the weights' dtype, then its expand); bit for bit
on integer data; bit for bit equal to the two-call GPU path (shrink, then
expand) where the shrink takes its 64-token form; and on the named fused
QKV and gate/up workloads at full size through that chain, each call
compared with the oracle over the whole output."""
import numpy as np
import pytest

import oracle
import sgmv_workloads as W
from gpu_util import (DeviceFused, assert_fused_parity, assert_parity, assert_shrink_parity,
                      to_host_bits)

pytestmark = pytest.mark.gpu

LENS = [70, 0, 129, 5, 64, 1, 200, 33]
IDX = [1, 0, -1, 2, 0, 1, 2, -1]


@pytest.mark.parametrize("K,slices,dts,add,scale", [
    (8, [(0, 64)], ("bf16", "bf16", "bf16"), False, 1.0),
    (16, [(8, 296), (320, 72)], ("f16", "f16", "f16"), True, 0.5),
    (24, [(0, 256)], ("f32", "bf16", "bf16"), True, 1.0),
    (32, [(0, 512), (512, 128), (640, 128)], ("bf16", "bf16", "bf16"), True, 1.0),
    (40, [(16, 200)], ("bf16", "bf16", "f32"), False, 2.0),
    (64, [(0, 1000), (1000, 1000)], ("bf16", "bf16", "bf16"), False, 1.0),
    (64, [(0, 264), (272, 8), (288, 256)], ("f16", "f16", "f32"), True, 1.0),
    (128, [(0, 520)], ("bf16", "bf16", "bf16"), True, 0.25),
    (128, [(0, 256), (256, 128)], ("f32", "f16", "f16"), False, 1.0),
    (8, [(0, 40), (40, 40), (80, 40)], ("f16", "f16", "bf16"), True, 1.0),   # 3 k tiles: no wave grid
])
def test_fused_parity(K, slices, dts, add, scale):
    x_dt, w_dt, o_dt = dts
    H_out = max(o + n for o, n in slices) + 8
    wl = W.fused_custom(LENS, IDX, H=1000, K=K, L=3, slices=slices, H_out=H_out, x_dtype=x_dt,
                        w_dtype=w_dt, out_dtype=o_dt, add=add, scale=scale, seed=K + len(slices))
    df = DeviceFused(wl)
    assert assert_fused_parity(wl, to_host_bits(df.run())) > 0


@pytest.mark.parametrize("K,ns,dts,add", [
    (8, 3, ("bf16", "bf16", "f32"), True),
    (8, 1, ("f16", "f16", "f16"), False),
    (64, 2, ("bf16", "bf16", "f32"), False),
    (32, 3, ("f32", "bf16", "f32"), True),
    (128, 2, ("f16", "f16", "f32"), True),
])
def test_fused_integer_data_bit_exact(K, ns, dts, add):
    # x, lora_A, lora_B in [-2, 2], hidden 16: projections |y| <= 64 are exact
    # in either 16-bit type; outputs |out| <= 8 + 128 K are exact in f32, and
    # in f16 (integers up to 2048) for rank 8
    x_dt, w_dt, o_dt = dts
    sl = [(64 * i, 48) for i in range(ns)]
    wl = W.fused_custom(LENS, IDX, H=16, K=K, L=3, slices=sl, H_out=64 * ns, x_dtype=x_dt,
                        w_dtype=w_dt, out_dtype=o_dt, add=add, values="int", seed=K * ns)
    df = DeviceFused(wl)
    assert assert_fused_parity(wl, to_host_bits(df.run()), exact=True) > 0


# From 64 units of 64 tokens (129 for ranks up to 16) the shrink takes its
# 64-token (split-T) form, whose sums the fused kernel reproduces: the
# results are then identical.
BIG_LENS = [1500, 3, 2000, 17, 0, 900, 1, 64, 65, 130]
BIG_IDX = [1, 0, 2, -1, 1, 0, 2, 1, -1, 0]


@pytest.mark.parametrize("K,slices,dts,add", [
    (16, [(0, 512)], ("bf16", "bf16", "bf16"), True),
    (32, [(0, 256), (256, 128), (384, 128)], ("bf16", "bf16", "bf16"), True),
    (64, [(0, 768), (768, 768)], ("bf16", "bf16", "bf16"), False),
    (128, [(8, 256)], ("f16", "f16", "f32"), True),
    (24, [(0, 136)], ("f32", "bf16", "f32"), False),
])
def test_fused_bit_identical_to_two_calls(K, slices, dts, add):
    x_dt, w_dt, o_dt = dts
    H_out = max(o + n for o, n in slices)
    lens = [2 * n for n in BIG_LENS] if K <= 16 else BIG_LENS
    wl = W.fused_custom(lens, BIG_IDX, H=512, K=K, L=3, slices=slices, H_out=H_out,
                        x_dtype=x_dt, w_dtype=w_dt, out_dtype=o_dt, add=add, seed=K)
    assert -(-wl.T // 64) >= (129 if K <= 16 else 64)
    df = DeviceFused(wl)
    fused = to_host_bits(df.run())
    _, two = df.run_two()
    assert np.array_equal(fused, to_host_bits(two)), "fused call differs from shrink + expand"
    assert assert_fused_parity(wl, fused) > 0


# Below 64 units of 64 tokens (129 for ranks up to 16) the shrink takes its
# 16-token (split-H) form, and so does the fused call: its 16-row units,
# each expanded over one of several column groups, reproduce the
# workspace-free two calls bit for bit.
SMALL_CASES = [
    # few units, 16 column tiles: one column group per tile
    (16, [(0, 4096)], ("bf16", "bf16", "bf16"), True, [20, 7, 33], [0, 1, -1], 1.0),
    # QKV-like, 6 column tiles over three slices
    (32, [(0, 1024), (1024, 256), (1280, 256)], ("bf16", "bf16", "bf16"), True, LENS, IDX, 1.0),
    (64, [(0, 2048), (2048, 2048)], ("f16", "f16", "f32"), False, LENS, IDX, 0.5),
    (128, [(0, 520)], ("f32", "bf16", "bf16"), True, LENS, IDX, 1.0),
    (8, [(0, 40), (40, 40), (80, 40)], ("f16", "f16", "bf16"), True, LENS, IDX, 2.0),
    (24, [(8, 264)], ("f32", "f16", "f16"), False, LENS, IDX, 1.0),
    # about 160 active units, more than half the compute units: one column
    # group each
    (16, [(0, 512), (512, 256)], ("bf16", "bf16", "bf16"), True, [1000, 1500, 3, 900],
     [2, 0, 1, -1], 1.0),
    # a decode step: one-token segments
    (16, [(0, 1024), (1024, 256)], ("bf16", "bf16", "bf16"), True, [1] * 200,
     [(i * 7) % 5 - 1 for i in range(200)], 1.0),
    # rank 16 between 64 and 128 units of 64 tokens (split-H up to 128):
    # about 460 units of 16, more than the compute units, several per
    # workgroup
    (16, [(0, 512), (512, 256), (768, 256)], ("bf16", "bf16", "f32"), True,
     [3000, 2500, 7, 1900], [1, 0, -1, 3], 1.0),
]


@pytest.mark.parametrize("K,slices,dts,add,lens,idx,scale", SMALL_CASES)
def test_fused_small_batches_bit_identical_to_two_calls(K, slices, dts, add, lens, idx, scale):
    x_dt, w_dt, o_dt = dts
    H_out = max(o + n for o, n in slices) + 8
    wl = W.fused_custom(lens, idx, H=1000 if K != 16 else 4096, K=K, L=5, slices=slices,
                        H_out=H_out, x_dtype=x_dt, w_dtype=w_dt, out_dtype=o_dt, add=add,
                        scale=scale, seed=K + len(slices) + len(lens))
    assert -(-wl.T // 64) < (129 if K <= 16 else 64)
    df = DeviceFused(wl)
    fused = to_host_bits(df.run())
    _, two = df.run_two()
    assert np.array_equal(fused, to_host_bits(two)), "fused call differs from shrink + expand"
    assert assert_fused_parity(wl, fused) > 0


@pytest.mark.parametrize("name", ["fused_q_proj", "fused_decode_qkv"])
def test_fused_small_named_workloads(name):
    """The short-prefill and decode workloads: equal to the two-call path bit
    for bit and within the fused tolerance of the oracle over every
    element."""
    wl = W.FUSED_WORKLOADS[name](0)
    df = DeviceFused(wl)
    fused = to_host_bits(df.run())
    _, two = df.run_two()
    assert np.array_equal(fused, to_host_bits(two)), "fused call differs from shrink + expand"
    assert assert_fused_parity(wl, fused) > 0


def test_fused_edge_layouts():
    # all -1, then fewer tokens than one unit, then a gap-and-order layout
    wl = W.fused_custom([5, 7], [-1, -1], H=64, K=16, L=2, slices=[(0, 64)], H_out=64, seed=1)
    df = DeviceFused(wl)
    assert np.array_equal(to_host_bits(df.run()), wl.out0)
    wl = W.fused_custom([3], [1], H=64, K=16, L=2, slices=[(0, 64)], H_out=64, add=True, seed=2)
    assert assert_fused_parity(wl, to_host_bits(DeviceFused(wl).run())) > 0
    wl = W.fused_custom([6, 17, 3, 40, 2], [1, 0, 1, 1, -1], H=256, K=32, L=2,
                        slices=[(24, 96), (128, 64)], H_out=200, start=[90, 3, 60, 20, 70], T=100,
                        add=True, seed=3)
    assert assert_fused_parity(wl, to_host_bits(DeviceFused(wl).run())) > 0


def test_fused_strided_inputs_and_output():
    wl = W.fused_custom([40, 25], [0, 1], H=128, K=32, L=2, slices=[(0, 64), (64, 64)],
                        H_out=128, add=True, seed=4, x_pad=8, out_pad=16)
    assert assert_fused_parity(wl, to_host_bits(DeviceFused(wl).run())) > 0


def test_fused_many_segments_unordered_table():
    # more than 512 segments: the segment table stays in index order
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 6, size=700).tolist()
    idx = rng.integers(-1, 4, size=700).tolist()
    wl = W.fused_custom(lens, idx, H=64, K=16, L=4, slices=[(0, 48), (48, 48)], H_out=96,
                        add=True, seed=5)
    assert assert_fused_parity(wl, to_host_bits(DeviceFused(wl).run())) > 0


@pytest.mark.parametrize("name", ["fused_qkv", "fused_gate_up"])
def test_fused_named_workloads(name):
    """Full size, through the chain: the two-call path's projection is
    compared with the oracle's shrink and its output with the oracle's
    expand of that projection, over every element; the fused call must
    equal the two-call path bit for bit."""
    wl = W.FUSED_WORKLOADS[name](0)
    df = DeviceFused(wl)
    fused = to_host_bits(df.run())
    ys, two = df.run_two()
    assert np.array_equal(fused, to_host_bits(two)), "fused call differs from shrink + expand"
    ys_bits = [to_host_bits(y) for y in ys]
    sw = W.ShrinkWorkload(name, wl.x, wl.x_dtype, wl.lora_a, wl.w_dtype,
                          [np.zeros_like(y) for y in ys_bits], wl.w_dtype, wl.start, wl.lens,
                          wl.idx, wl.scale, wl.K, wl.L, wl.seed)
    assert assert_shrink_parity(sw, ys_bits) > 0
    ew = W.Workload(name, [W.SliceInput(y, wl.w_dtype, b, wl.w_dtype, off)
                           for y, b, off in zip(ys_bits, wl.lora_b, wl.offsets)],
                    wl.out0, wl.out_dtype, wl.start, wl.lens, wl.idx, wl.add, wl.K, wl.L, wl.seed)
    rep = assert_parity(ew, fused)
    t_act = int(wl.lens[wl.active_mask()].sum())
    assert rep.checked_values == t_act * sum(b.shape[1] for b in wl.lora_b)


@pytest.mark.parametrize("units", [255, 256, 257])
def test_fused_unit_assignment_around_the_compute_unit_count(units):
    """`units` segments of 64 tokens, one fused unit each, in a grid sized from
    ceil(T / 64) + segments: both branches of the unit assignment (even
    shares per XCD while every unit has a compute unit; XCD after XCD
    beyond)."""
    lens = [64] * units
    idx = [i % 5 for i in range(units)]
    wl = W.fused_custom(lens, idx, H=128, K=32, L=5, slices=[(0, 256), (256, 128)], H_out=400,
                        add=units % 2 == 1, seed=units)
    assert assert_fused_parity(wl, to_host_bits(DeviceFused(wl).run())) > 0
