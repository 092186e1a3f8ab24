"""GPU parity on the five named workloads at full size, through the C ABI, in
the same launch configuration the benchmark times.

Small workloads are compared element by element with the CPU oracle over
the whole output.  The two large ones (gate/up MLP, skewed batch) are
compared on sampled rows -- every segment's first and last row plus random
rows -- with the oracle's streaming comparator, and on the whole output for
the bit-exact property that every element outside the written region keeps
its prior bits (checked on the device).
"""
import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceWorkload, assert_parity, to_host_bits

pytestmark = pytest.mark.gpu


def assert_untouched_on_device(dw, out):
    """Every element outside (active rows x slice windows) equals its prior bits."""
    import torch
    wl = dw.wl
    act = torch.zeros(wl.T, dtype=torch.bool)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            act[s:s + n] = True
    act = act.to(out.device)
    cols = torch.zeros(wl.H, dtype=torch.bool)
    for s in wl.slices:
        cols[s.offset:s.offset + s.N] = True
    cols = cols.to(out.device)
    ib = torch.int32 if out.dtype == torch.float32 else torch.int16
    same = out.view(ib) == dw.out0.view(ib)
    written = act[:, None] & cols[None, :]
    bad = (~same & ~written).sum().item()
    assert bad == 0, f"{bad} elements outside the written region changed"


def sample_rows(wl, n_random=256, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.integers(0, wl.T, size=n_random).tolist())
    for s, n in zip(wl.start, wl.lens):
        if n > 0:
            rows.update([int(s), int(s + n - 1)])
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_ref(seed):
    wl = W.tiny_ref(seed)
    dw = DeviceWorkload(wl)
    out = dw.run_single(dw.fresh_out())
    bits = to_host_bits(out)
    assert_parity(wl, bits)
    assert np.array_equal(bits[4:], wl.out0[4:])          # index -1 segment untouched


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_llama7b_q_proj(seed):
    wl = W.llama7b_q_proj(seed)
    dw = DeviceWorkload(wl)
    out = dw.run_single(dw.fresh_out())
    assert_parity(wl, to_host_bits(out))


@pytest.mark.parametrize("shared_input", [False, True])
def test_gqa_qkv_single_and_multi(shared_input):
    wl = W.gqa_qkv(0, shared_input=shared_input)
    dw = DeviceWorkload(wl)
    three = to_host_bits(dw.run_all_single(dw.fresh_out()))
    fused = to_host_bits(dw.run_multi(dw.fresh_out()))
    assert np.array_equal(three, fused), "multi-slice differs from three single-slice calls"
    assert_parity(wl, fused)


def test_mlp_gate_up():
    wl = W.mlp_gate_up(0)
    dw = DeviceWorkload(wl)
    out = dw.run_single(dw.fresh_out())
    assert_untouched_on_device(dw, out)
    rows = sample_rows(wl)
    bits = to_host_bits(out[torch_rows(rows, out.device)])
    sub = subset_workload(wl, rows)
    assert_parity(sub, bits)


def test_skewed_mixed():
    wl = W.skewed_mixed(0)
    dw = DeviceWorkload(wl)
    out = dw.run_single(dw.fresh_out())
    assert_untouched_on_device(dw, out)
    rows = sample_rows(wl)
    long_seg = int(np.argmax(wl.lens))
    s0 = int(wl.start[long_seg])
    rows = np.union1d(rows, np.arange(s0, s0 + 64))     # a run inside the long segment
    bits = to_host_bits(out[torch_rows(rows, out.device)])
    assert_parity(subset_workload(wl, rows), bits)


def torch_rows(rows, device):
    import torch
    return torch.from_numpy(rows).to(device)


def subset_workload(wl, rows):
    """The workload restricted to `rows` (in order): each kept row becomes a
    one-row segment with its original adapter, so the oracle's comparator
    sees exactly those rows."""
    row_adapter = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if a >= 0 and n > 0:
            row_adapter[s:s + n] = a
    k = len(rows)
    slices = [W.SliceInput(np.ascontiguousarray(s.x[rows]), s.x_dtype, s.w, s.w_dtype, s.offset)
              for s in wl.slices]
    return W.Workload(wl.name + "[rows]", slices, np.ascontiguousarray(wl.out0[rows]),
                      wl.out_dtype, np.arange(k, dtype=np.int64), np.ones(k, dtype=np.int64),
                      row_adapter[rows], wl.add, wl.K, wl.L, wl.seed)
