"""GPU parity of the LoRA-A projection (shrink) entry points, sgmv_shrink and
sgmv_shrink_multi_slice, against the CPU oracle (the projection that produces
the expand's inputs; wiki page "Implementation: Predibase Lorax SGMV Expand
Slice Kernel", I/O Contract, Inputs; Usage Examples).

Cases span several 16-row tiles and ragged tails, ranks that are not a
multiple of 16 (partial k tiles), hidden sizes that are not a multiple of 32
(partial hidden steps) or not of 8 (the generic kernel), strided rows, every
dtype combination, one to eight slices (split launches past 16 k tiles),
segment tables ordered by adapter, and the named workloads at full size on
sampled rows."""
import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceShrink, assert_shrink_parity, to_host_bits

pytestmark = pytest.mark.gpu


def run_and_check(wl, rows=None, multi=True, exact=False):
    print(f"case {wl.name} T={wl.T} H={wl.H} K={wl.K} slices={len(wl.lora_a)} "
          f"dtypes={wl.x_dtype}/{wl.a_dtype}/{wl.out_dtype}", flush=True)
    dw = DeviceShrink(wl)
    outs = [to_host_bits(o) for o in dw.run(multi=multi)]
    return assert_shrink_parity(wl, outs, rows=rows, exact=exact)


def ragged(seed, B, max_len, L, p_off=0.2):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, max_len + 1, size=B)
    idx = rng.integers(0, L, size=B)
    idx[rng.random(B) < p_off] = -1
    return lens.tolist(), idx.tolist()


@pytest.mark.parametrize("H,K,slices,dts,scale", [
    (4096, 16, 1, ("bf16", "bf16", "bf16"), 2.0),
    (1000, 24, 1, ("f16", "f16", "f32"), 1.0),     # partial hidden step, partial k tile
    (64, 8, 1, ("f32", "bf16", "bf16"), 0.5),      # float32 input, two hidden steps
    (8192, 128, 1, ("f16", "f16", "f16"), 1.0),    # 8 k tiles
    (512, 256, 1, ("bf16", "bf16", "f32"), 1.0),   # 16 k tiles
    (2048, 32, 3, ("bf16", "bf16", "bf16"), 1.0),  # fused QKV: 6 of 8 k tiles live
    (1024, 64, 2, ("f32", "f16", "f32"), 0.25),    # gate/up
    (256, 64, 8, ("bf16", "bf16", "bf16"), 1.0),   # 32 k tiles: two launches
    (384, 128, 3, ("f16", "f16", "bf16"), 3.0),    # 24 k tiles: two launches
    (40, 8, 1, ("f16", "f16", "f16"), 1.0),        # hidden 40: one partial step
])
def test_shrink_parity(H, K, slices, dts, scale):
    lens, idx = ragged(H + K + slices, 12, 70, 5)
    x_dt, a_dt, o_dt = dts
    wl = W.shrink_custom(lens, idx, H=H, K=K, L=5, slices=slices, x_dtype=x_dt, a_dtype=a_dt,
                         out_dtype=o_dt, scale=scale, seed=H + K)
    assert run_and_check(wl) > 0


@pytest.mark.parametrize("H,K,slices,dts,scale", [
    (4096, 16, 1, ("bf16", "bf16", "f32"), 1.0),
    (1000, 24, 2, ("f16", "f16", "f16"), 2.0),
    (8192, 128, 1, ("f32", "f16", "bf16"), 0.5),
    (2048, 32, 3, ("bf16", "bf16", "bf16"), 1.0),
    (100, 16, 1, ("bf16", "bf16", "f32"), 1.0),    # generic kernel
    (96, 7, 1, ("f16", "f16", "f32"), 4.0),        # generic kernel
])
def test_shrink_integer_data_bit_exact(H, K, slices, dts, scale):
    """x and lora_A in [-3, 3]: every fp32 partial sum is an exact integer
    (|sum| <= 9 H < 2^24), so in any summation order the result is the exact
    value rounded once, the oracle's bits.  A dropped, repeated or misplaced
    product changes the sum and fails this."""
    lens, idx = ragged(H + 5 * K, 10, 50, 4)
    x_dt, a_dt, o_dt = dts
    wl = W.shrink_custom(lens, idx, H=H, K=K, L=4, slices=slices, x_dtype=x_dt, a_dtype=a_dt,
                         out_dtype=o_dt, scale=scale, values="int", seed=H + K + 1)
    assert run_and_check(wl, exact=True) > 0


@pytest.mark.parametrize("H,K,x_pad,out_pad,dts", [
    (100, 16, 0, 0, ("bf16", "bf16", "bf16")),     # hidden % 8 != 0: generic
    (96, 7, 0, 0, ("f16", "f16", "f32")),          # rank 7: generic
    (128, 16, 3, 0, ("bf16", "bf16", "bf16")),     # misaligned input rows: generic
    (128, 16, 8, 8, ("bf16", "bf16", "bf16")),     # strided but aligned: fast
    (256, 32, 0, 5, ("f32", "bf16", "f16")),       # misaligned output rows: generic
    (72, 24, 4, 4, ("f32", "f16", "f32")),         # strided float32 rows, aligned: fast
])
def test_shrink_strides_and_generic(H, K, x_pad, out_pad, dts):
    lens, idx = ragged(H * 3 + K, 9, 40, 3)
    x_dt, a_dt, o_dt = dts
    wl = W.shrink_custom(lens, idx, H=H, K=K, L=3, x_dtype=x_dt, a_dtype=a_dt, out_dtype=o_dt,
                         x_pad=x_pad, out_pad=out_pad, seed=H + 7 * K)
    assert run_and_check(wl) > 0


def test_shrink_multi_slice_equals_single_calls():
    lens, idx = ragged(3, 20, 90, 6)
    wl = W.shrink_custom(lens, idx, H=2048, K=32, L=6, slices=3, seed=3)
    dw = DeviceShrink(wl)
    a = [to_host_bits(o) for o in dw.run(multi=True)]
    b = [to_host_bits(o) for o in dw.run(multi=False)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_shrink_adapter_ordered_table():
    """300 short segments (the table is ordered by adapter for 128..512
    segments) with shuffled starts."""
    rng = np.random.default_rng(9)
    B = 300
    lens = rng.integers(1, 12, size=B)
    order = rng.permutation(B)
    start = np.zeros(B, dtype=np.int64)
    pos = 0
    for b in order:
        start[b] = pos
        pos += int(lens[b])
    idx = rng.integers(-1, 20, size=B)
    wl = W.shrink_custom(lens, idx, H=512, K=16, L=20, start=start, T=pos, seed=9)
    assert run_and_check(wl) > 0



@pytest.mark.parametrize("B,max_len", [(16, 30), (17, 30), (33, 30), (64, 30), (65, 30),
                                       (49, 200), (64, 200), (65, 200)])
def test_shrink_segment_counts_around_the_wave_scan(B, max_len):
    """Segment counts at the edges of the in-register table scan (16-lane
    rows, one wave of 64); the longer segments reach the 64-token units."""
    lens, idx = ragged(700 + B + max_len, B, max_len, 6)
    wl = W.shrink_custom(lens, idx, H=256, K=16, L=6, seed=B)
    assert run_and_check(wl) > 0


@pytest.mark.parametrize("L", [40, 1100])
def test_shrink_adapter_ordered_table_few_and_many_adapters(L):
    """300 segments ordered by adapter, over few or over many adapters."""
    rng = np.random.default_rng(300 + L)
    B = 300
    lens = rng.integers(1, 30, size=B)
    idx = rng.integers(-1, L, size=B)
    wl = W.shrink_custom(lens, idx, H=256, K=16, L=L, seed=12)
    assert run_and_check(wl) > 0

def test_shrink_long_segment_several_units_per_workgroup():
    """More 16-row tiles than the grid holds workgroups."""
    wl = W.shrink_custom([9000, 37, 1], [1, 0, 1], H=256, K=16, L=2, seed=10)
    assert run_and_check(wl) > 0


def test_shrink_out_of_range_index_is_skipped():
    """Index >= lora_num is outside the contract; the kernel skips such a
    segment without touching its rows (the oracle sees it as -1)."""
    wl = W.shrink_custom([20, 30, 10], [0, 1, 1], H=128, K=16, L=2, seed=11)
    import torch
    dw = DeviceShrink(wl)
    bad_idx = torch.tensor([0, 5, 1], dtype=torch.int64, device="cuda")
    outs = [to_host_bits(o) for o in dw.run(idx=bad_idx)]
    assert assert_shrink_parity(wl, outs, idx=np.array([0, -1, 1])) > 0


def test_shrink_all_without_adapter_touch_nothing():
    wl = W.shrink_custom([5, 9, 4], [-1, -1, -1], H=128, K=16, L=2, seed=12)
    dw = DeviceShrink(wl)
    outs = [to_host_bits(o) for o in dw.run()]
    assert np.array_equal(outs[0], wl.outs0[0])


def test_shrink_tiny_worked_example_segments():
    assert run_and_check(W.shrink_tiny(0)) > 0


@pytest.mark.parametrize("name,sample", [
    ("shrink_q_proj", None), ("shrink_qkv", 384), ("shrink_gate_up", 256),
    ("shrink_skewed", 256)])
def test_shrink_named_workloads(name, sample):
    """Full-size workloads; large ones are checked on a seeded sample of rows
    (every row's untouched check still runs)."""
    wl = W.SHRINK_WORKLOADS[name](0)
    rows = None
    if sample is not None:
        rng = np.random.default_rng(1)
        rows = np.sort(rng.choice(wl.T, size=sample, replace=False))
        rows = np.unique(np.concatenate([rows, [0, wl.T - 1]]))
    assert run_and_check(wl, rows=rows) > 0


# Batches of at least 256 64-token units take the split-T kernels (64-token
# units, lora_A shared through LDS); smaller ones the split-H kernels.
SPLIT_T_LENS = [5000, 3, 7000, 17, 0, 4500, 1, 64, 65]
SPLIT_T_IDX = [1, 0, 2, -1, 1, 0, 2, 1, -1]


@pytest.mark.parametrize("H,K,slices,dts,scale", [
    (256, 16, 1, ("bf16", "bf16", "bf16"), 1.0),
    (1000, 24, 2, ("f16", "f16", "f32"), 0.5),     # partial hidden step, partial k tile
    (64, 128, 1, ("f32", "bf16", "bf16"), 1.0),
    (512, 32, 3, ("bf16", "bf16", "bf16"), 2.0),   # fused QKV shape
    (96, 256, 1, ("f16", "f16", "f16"), 1.0),      # 16 k tiles
    (40, 8, 3, ("f32", "f16", "f32"), 1.0),
    (128, 64, 5, ("bf16", "bf16", "f32"), 1.0),    # 5 slices: launches of 2 and 3
    (256, 32, 1, ("bf16", "bf16", "bf16"), 1.0),   # 2 k tiles: one token tile per wave
    (128, 16, 2, ("f16", "f16", "f16"), 1.0),      # 2 k tiles over two slices
])
def test_shrink_split_t_parity(H, K, slices, dts, scale):
    x_dt, a_dt, o_dt = dts
    wl = W.shrink_custom(SPLIT_T_LENS, SPLIT_T_IDX, H=H, K=K, L=3, slices=slices, x_dtype=x_dt,
                         a_dtype=a_dt, out_dtype=o_dt, scale=scale, seed=H * K + slices)
    assert -(-wl.T // 64) >= 256
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(wl.T, size=3000, replace=False),
                                     np.arange(0, 200), np.arange(wl.T - 200, wl.T)]))
    assert run_and_check(wl, rows=rows) > 0


@pytest.mark.parametrize("H,K,slices,dts", [
    (256, 16, 1, ("bf16", "bf16", "f32")),
    (1000, 24, 3, ("f16", "f16", "bf16")),
    (72, 128, 2, ("f32", "bf16", "f32")),
])
def test_shrink_split_t_integer_data_bit_exact(H, K, slices, dts):
    x_dt, a_dt, o_dt = dts
    wl = W.shrink_custom(SPLIT_T_LENS, SPLIT_T_IDX, H=H, K=K, L=3, slices=slices, x_dtype=x_dt,
                         a_dtype=a_dt, out_dtype=o_dt, values="int", seed=H + K)
    assert run_and_check(wl, exact=True) > 0


def test_shrink_multi_slice_with_a_misaligned_output_equals_single_calls():
    """A slice whose output rows are not 16-byte aligned runs on the generic
    kernel; the other slices of the same call keep their fast kernel, so
    every slice equals its own single call bit for bit."""
    import torch
    import segmented_gather_gemm_amd as sg
    lens, idx = ragged(21, 14, 80, 4)
    wl = W.shrink_custom(lens, idx, H=1024, K=32, L=4, slices=3, seed=21)
    dw = DeviceShrink(wl)
    wide = torch.zeros((wl.T, wl.K + 3), dtype=torch.bfloat16, device="cuda")
    outs = dw.fresh_outs()
    wide[:, :wl.K] = outs[1]
    outs[1] = wide[:, :wl.K]                       # row stride 35 elements: misaligned
    sg.sgmv_shrink_multi_slice(dw.x, list(zip(dw.a, outs)), dw.start, dw.lens, dw.idx,
                               wl.batches, wl.max_seq_len, wl.scale)
    for i in range(3):
        alone = dw.fresh_outs()[i]
        if i == 1:
            w2 = torch.zeros_like(wide)
            w2[:, :wl.K] = alone
            alone = w2[:, :wl.K]
        sg.sgmv_shrink(dw.x, dw.a[i], alone, dw.start, dw.lens, dw.idx, wl.batches,
                       wl.max_seq_len, wl.scale)
        assert np.array_equal(to_host_bits(outs[i]), to_host_bits(alone)), i
    assert assert_shrink_parity(wl, [to_host_bits(o) for o in outs]) > 0
