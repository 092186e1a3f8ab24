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


def run_and_check(wl, rows=None, multi=True, exact=False, workspace=True):
    print(f"case {wl.name} T={wl.T} H={wl.H} K={wl.K} slices={len(wl.lora_a)} "
          f"dtypes={wl.x_dtype}/{wl.a_dtype}/{wl.out_dtype} workspace={workspace}", flush=True)
    dw = DeviceShrink(wl)
    outs = [to_host_bits(o) for o in dw.run(multi=multi, workspace=workspace)]
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


@pytest.mark.parametrize("name", ["shrink_q_proj", "shrink_qkv", "shrink_gate_up",
                                  "shrink_skewed"])
def test_shrink_named_workloads(name):
    """Full-size workloads, every row compared with the oracle."""
    wl = W.SHRINK_WORKLOADS[name](0)
    assert run_and_check(wl) > 0


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
    # slice 1 ran on the generic kernel: its summation depth is the hidden size
    assert assert_shrink_parity(wl, [to_host_bits(o) for o in outs], depth=wl.H) > 0


@pytest.mark.parametrize("slices,dts", [(1, ("bf16", "bf16", "f32")), (3, ("f16", "f16", "f16"))])
def test_shrink_rank16_split_h_up_to_128_units(slices, dts):
    """Ranks up to 16 keep the 16-token (split-H) form through 128 units of
    64 tokens: 116 units here, several 16-token units per workgroup; every
    row compared with the oracle, and integer data bit for bit."""
    x_dt, a_dt, o_dt = dts
    lens, idx = [3000, 2500, 7, 1900], [1, 0, -1, 2]
    wl = W.shrink_custom(lens, idx, H=2048, K=16, L=3, slices=slices, x_dtype=x_dt,
                         a_dtype=a_dt, out_dtype=o_dt, seed=40 + slices)
    assert 64 < -(-wl.T // 64) < 129
    assert run_and_check(wl) > 0
    wi = W.shrink_custom(lens, idx, H=256, K=16, L=3, slices=slices, x_dtype=x_dt,
                         a_dtype=a_dt, out_dtype=o_dt, values="int", seed=50 + slices)
    assert run_and_check(wi, exact=True) > 0


@pytest.mark.parametrize("units", [255, 256, 257])
def test_shrink_unit_assignment_around_the_compute_unit_count(units):
    """`units` segments of 64 tokens, each one split-T unit, in a grid of about
    twice as many workgroups (the host sizes it from ceil(T / 64) + segments):
    without a workspace, up to the compute unit count the units are spread
    evenly over the XCDs, beyond it they fill XCD after XCD (unit_span in
    sgmv_limits.h).  Every row of every unit is compared with the oracle."""
    lens = [64] * units
    idx = [i % 7 for i in range(units)]  # every segment active: exactly `units` units
    wl = W.shrink_custom(lens, idx, H=256, K=64, L=7, slices=2, x_dtype="bf16", a_dtype="bf16",
                         out_dtype="f32", seed=units)
    assert run_and_check(wl, workspace=None) > 0


def compute_units():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def units_workload(units, seed, values="normal", H=1024, K=64, slices=2,
                   dts=("bf16", "bf16", "f32")):
    """`units` active segments of 64 tokens (exactly that many split-T
    units), adapters cycling over 7."""
    lens = [64] * units
    idx = [i % 7 for i in range(units)]
    return W.shrink_custom(lens, idx, H=H, K=K, L=7, slices=slices, x_dtype=dts[0],
                           a_dtype=dts[1], out_dtype=dts[2], values=values, seed=seed)


# Units beyond the compute units C: 1 (8 parts each), C/6 (6 parts), C/4 (4),
# C/2 (2), C/2 + 1 and C (one part each: unit_span instead), C + 1 (more than
# 2 C units: unit_span).
BALANCE_EXTRA = [1, 42, 64, 128, 129, 256, 257]


@pytest.mark.parametrize("extra", BALANCE_EXTRA)
def test_shrink_balanced_parts_around_twice_the_compute_units(extra):
    """With the workspace, C < U <= 2 C units run as one whole unit per
    compute unit plus the other units cut into hidden parts whose fp32 sums
    are added through the workspace (limits::part_plan); every row of every
    unit is compared with the oracle."""
    C = compute_units()
    wl = units_workload(C + extra, seed=extra)
    assert run_and_check(wl) > 0


# Small split-T batches (at least 64 units of 64 tokens): C/4 units (4 parts
# each), about C/3 (3), C/2.56 and C/2 (2), C/2 + 1 (one part: unit_span).
SMALL_UNITS = [64, 85, 100, 128, 129]


@pytest.mark.parametrize("units", SMALL_UNITS)
def test_shrink_balanced_small_batches_every_unit_in_parts(units):
    """With the workspace and at most C / 2 units, every unit is cut into
    hidden parts so that the idle compute units share the work
    (limits::part_plan); every row compared with the oracle."""
    C = compute_units()
    wl = units_workload(units * C // 256, seed=500 + units)
    assert run_and_check(wl) > 0


@pytest.mark.parametrize("units", [64, 100])
def test_shrink_balanced_small_batches_integer_and_multi_slice(units):
    """Small balanced batches: integer data bit for bit equal to the call
    without a workspace and to the oracle, and a three-slice call equal to
    its single calls on random data."""
    C = compute_units()
    n = units * C // 256
    wl = units_workload(n, seed=600 + units, values="int", H=1000, K=24, slices=3,
                        dts=("f16", "f16", "bf16"))
    dw = DeviceShrink(wl)
    bal = [to_host_bits(o) for o in dw.run(workspace=True)]
    plain = [to_host_bits(o) for o in dw.run(workspace=None)]
    for a, b in zip(bal, plain):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wl, bal, exact=True) > 0
    wl2 = units_workload(n, seed=700 + units, H=4096, K=32, slices=3,
                         dts=("bf16", "bf16", "bf16"))
    dw2 = DeviceShrink(wl2)
    multi = [to_host_bits(o) for o in dw2.run(multi=True)]
    single = [to_host_bits(o) for o in dw2.run(multi=False)]
    for a, b in zip(multi, single):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wl2, multi) > 0


@pytest.mark.parametrize("units,K,H", [(16, 128, 8192), (40, 256, 4096), (63, 72, 2048)])
def test_shrink_wide_ranks_take_split_t_from_16_units_with_a_workspace(units, K, H):
    """Ranks above 64 take the balanced split-T kernel from 16 units of 64
    tokens when a workspace comes with the call (split-H without one): both
    match the oracle, and on integer data they agree bit for bit."""
    C = compute_units()
    n = max(16, units * C // 256)
    wl = units_workload(n, seed=800 + K, H=H, K=K, slices=1, dts=("f16", "f16", "f16"))
    assert run_and_check(wl) > 0
    assert run_and_check(wl, workspace=None) > 0
    wi = units_workload(n, seed=900 + K, values="int", H=H, K=K, slices=1,
                        dts=("bf16", "bf16", "f32"))
    dw = DeviceShrink(wi)
    bal = [to_host_bits(o) for o in dw.run(workspace=True)]
    plain = [to_host_bits(o) for o in dw.run(workspace=None)]
    for a, b in zip(bal, plain):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wi, bal, exact=True) > 0


@pytest.mark.parametrize("extra", [1, 42, 128, 129])
def test_shrink_balanced_integer_data_bit_exact_and_equal_without_workspace(extra):
    """On integer-valued data every fp32 partial sum is exact, so the
    balanced call, the call without a workspace and the oracle agree bit for
    bit (hidden 1000: a partial last step, and parts of unequal length)."""
    C = compute_units()
    wl = units_workload(C + extra, seed=100 + extra, values="int", H=1000, K=24, slices=3,
                        dts=("f16", "f16", "bf16"))
    dw = DeviceShrink(wl)
    bal = [to_host_bits(o) for o in dw.run(workspace=True)]
    plain = [to_host_bits(o) for o in dw.run(workspace=None)]
    for a, b in zip(bal, plain):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wl, bal, exact=True) > 0


@pytest.mark.parametrize("units,K,slices", [(None, 64, 2), (64, 32, 3), (16, 128, 1)])
def test_shrink_balanced_float32_inputs(units, K, slices):
    """float32 inputs (rounded to the weight dtype on the way into LDS) on
    the balanced paths: C + 42 units (parts beside whole units), 64 units
    (every unit in parts) and 16 units of rank 128 (split-T below 64 units),
    against the oracle, and on integer data bit for bit equal to the call
    without a workspace."""
    C = compute_units()
    n = C + 42 if units is None else max(16, units * C // 256)
    wl = units_workload(n, seed=1000 + n + K, H=2048, K=K, slices=slices,
                        dts=("f32", "bf16", "f32"))
    assert run_and_check(wl) > 0
    wi = units_workload(n, seed=1100 + n + K, values="int", H=2048, K=K, slices=slices,
                        dts=("f32", "f16", "f32"))
    dw = DeviceShrink(wi)
    bal = [to_host_bits(o) for o in dw.run(workspace=True)]
    plain = [to_host_bits(o) for o in dw.run(workspace=None)]
    for a, b in zip(bal, plain):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wi, bal, exact=True) > 0


@pytest.mark.parametrize("target,seed", [(300, 1), (80, 2)])
def test_shrink_balanced_ragged_segments(target, seed):
    """Balanced batches built from ragged segments (1..200 tokens, so many
    units hold fewer than 64 rows), index -1 and empty segments among them:
    about `target` units on a 256-unit device (C + 44: parts beside whole
    units; 80: every unit in parts).  Every row is compared with the oracle
    and rows without an adapter keep their bits."""
    C = compute_units()
    rng = np.random.default_rng(seed)
    want = target * C // 256
    lens, idx, units = [], [], 0
    while units < want:
        n = int(rng.integers(0, 201))
        a = -1 if rng.random() < 0.12 else int(rng.integers(0, 9))
        lens.append(n)
        idx.append(a)
        if a >= 0:
            units += -(-n // 64)
    wl = W.shrink_custom(lens, idx, H=2048, K=48, L=9, slices=2, x_dtype="bf16",
                         a_dtype="bf16", out_dtype="f32", seed=1200 + seed)
    assert run_and_check(wl) > 0
    wi = W.shrink_custom(lens, idx, H=2048, K=48, L=9, slices=2, x_dtype="f16", a_dtype="f16",
                         out_dtype="f16", values="int", seed=1300 + seed)
    dw = DeviceShrink(wi)
    bal = [to_host_bits(o) for o in dw.run(workspace=True)]
    plain = [to_host_bits(o) for o in dw.run(workspace=None)]
    for a, b in zip(bal, plain):
        assert np.array_equal(a, b)
    assert assert_shrink_parity(wi, bal, exact=True) > 0


def test_shrink_balanced_multi_slice_equals_single_calls():
    """Part boundaries depend only on the hidden size and the part count, so
    a three-slice call (one launch of 6 k tiles) equals three single calls
    (2 k tiles each, another pipeline shape) bit for bit on random data."""
    C = compute_units()
    wl = units_workload(C + 42, seed=7, H=4096, K=32, slices=3, dts=("bf16", "bf16", "bf16"))
    dw = DeviceShrink(wl)
    a = [to_host_bits(o) for o in dw.run(multi=True)]
    b = [to_host_bits(o) for o in dw.run(multi=False)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert assert_shrink_parity(wl, a) > 0


def test_shrink_balanced_repeated_calls_and_a_callers_workspace():
    """Calls in a row on the shared workspace (each leaves its counters at
    zero for the next), a smaller batch after a larger one, and a caller's
    own zero-filled workspace all give the same results."""
    import torch
    import segmented_gather_gemm_amd as sg
    C = compute_units()
    big = units_workload(C + 30, seed=31)
    small = units_workload(C + 5, seed=32)
    dbig, dsmall = DeviceShrink(big), DeviceShrink(small)
    first = [to_host_bits(o) for o in dbig.run()]
    assert assert_shrink_parity(big, first) > 0
    assert assert_shrink_parity(small, [to_host_bits(o) for o in dsmall.run()]) > 0
    again = [to_host_bits(o) for o in dbig.run()]
    ws = torch.zeros(sg.shrink_workspace_bytes(), dtype=torch.uint8, device="cuda")
    own = [to_host_bits(o) for o in dbig.run(workspace=ws)]
    for x, y, z in zip(first, again, own):
        assert np.array_equal(x, y) and np.array_equal(x, z)
    counter_bytes = (4 * C + 255) // 256 * 256
    assert not bool(ws[:counter_bytes].any())  # the counters are back at zero


def test_shrink_workspace_size_and_alignment_checked():
    import ctypes
    import torch
    import segmented_gather_gemm_amd as sg
    C = compute_units()
    need = sg.shrink_workspace_bytes()
    assert need == (4 * C + 255) // 256 * 256 + C * 64 * 256 * 4
    wl = units_workload(C + 1, seed=3)
    dw = DeviceShrink(wl)
    ws = torch.zeros(need + 16, dtype=torch.uint8, device="cuda")
    for ptr, n, frag in ((ws.data_ptr(), need - 1, "hold"), (ws.data_ptr() + 8, need, "aligned")):
        out = dw.fresh_outs()[0]
        st = sg.lib.sgmv_shrink(sg._matrix(dw.x, "x"), sg._stack_a(dw.a[0], "a"),
                                sg._matrix(out, "out"), dw.start.data_ptr(), dw.lens.data_ptr(),
                                dw.idx.data_ptr(), wl.batches, wl.max_seq_len,
                                ctypes.c_float(wl.scale), ptr, n, None)
        assert st == sg.SGMV_ERR_INVALID_ARGUMENT
        assert frag in sg.lib.sgmv_last_error().decode()
