"""HIP-graph capture of the C-ABI calls: a captured sgmv_expand_slice /
sgmv_expand_multi_slice, sgmv_shrink / sgmv_shrink_multi_slice or
sgmv_fused_shrink_expand replayed several times, with eager work and
synchronisation between replays, gives the eager result on every replay
(the library records no memset or allocation, only kernel launches)."""
import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceWorkload, assert_parity, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("multi", [False, True])
def test_graph_replays_match_eager(multi):
    import torch
    extra = [(300, 70)] if multi else []
    wl = W.custom([40, 3, 0, 19, 70], [1, 0, 1, -1, 0], K=32, N=256, H=400, off=16, L=2,
                  add=True, seed=31, extra_slices=extra)
    dw = DeviceWorkload(wl)
    run = dw.run_multi if multi else dw.run_all_single
    eager = to_host_bits(run(dw.fresh_out()))
    assert_parity(wl, eager)
    out = dw.fresh_out()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(out)
    for replay in range(4):
        out.copy_(dw.out0)                       # eager reset between replays
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), eager), f"replay {replay}"
        other = to_host_bits(run(dw.fresh_out()))  # eager work in between
        torch.cuda.synchronize()
        assert np.array_equal(other, eager)


@pytest.mark.parametrize("multi,T", [(False, 300), (True, 300), (True, 5000)])
def test_shrink_graph_replays_match_eager(multi, T):
    """sgmv_shrink / sgmv_shrink_multi_slice captured once and replayed; T =
    5000 takes the split-T kernels, T = 300 the split-H ones."""
    import torch
    from gpu_util import DeviceShrink, assert_shrink_parity
    rng = np.random.default_rng(T)
    lens = rng.integers(1, 2 * T // 10, size=10)
    lens = (lens * T // lens.sum()).tolist()
    wl = W.shrink_custom(lens, [0, 1, -1, 2, 1, 0, 2, -1, 1, 0], H=512, K=32, L=3,
                         slices=3 if multi else 1, seed=T)
    dw = DeviceShrink(wl)
    eager = [to_host_bits(o) for o in dw.run(multi=multi)]
    assert assert_shrink_parity(wl, eager) > 0
    outs = dw.fresh_outs()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dw.run(outs, multi=multi)
    for replay in range(4):
        for o, o0 in zip(outs, dw.outs0):
            o.copy_(o0)                           # eager reset between replays
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(to_host_bits(o), eager[i]), f"replay {replay} slice {i}"
        other = [to_host_bits(o) for o in dw.run(multi=multi)]  # eager work in between
        torch.cuda.synchronize()
        for a, b in zip(other, eager):
            assert np.array_equal(a, b)


def test_shrink_balanced_graph_replays_match_eager():
    """A balanced split-T call (more 64-token units than compute units, parts
    added through the shared workspace) captured and replayed with eager
    calls in between: every replay leaves the workspace counters at zero for
    the next call, eager or replayed."""
    import torch
    from gpu_util import DeviceShrink, assert_shrink_parity
    C = torch.cuda.get_device_properties(0).multi_processor_count
    units = C + 42
    wl = W.shrink_custom([64] * units, [i % 5 for i in range(units)], H=1024, K=64, L=5,
                         slices=2, x_dtype="bf16", a_dtype="bf16", out_dtype="f32", seed=units)
    dw = DeviceShrink(wl)
    eager = [to_host_bits(o) for o in dw.run()]
    assert assert_shrink_parity(wl, eager) > 0
    outs = dw.fresh_outs()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dw.run(outs)
    for replay in range(4):
        for o, o0 in zip(outs, dw.outs0):
            o.copy_(o0)
        graph.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(to_host_bits(o), eager[i]), f"replay {replay} slice {i}"
        other = [to_host_bits(o) for o in dw.run()]
        torch.cuda.synchronize()
        for a, b in zip(other, eager):
            assert np.array_equal(a, b)


@pytest.mark.parametrize("add,large", [(False, False), (True, False), (True, True)])
def test_fused_graph_replays_match_eager(add, large):
    """sgmv_fused_shrink_expand captured once and replayed: a short batch
    (the 16-row form) and, with ``large``, a batch of more than 64 units of
    64 tokens (the 64-row form)."""
    import torch
    from gpu_util import DeviceFused, assert_fused_parity
    lens = [90, 3, 0, 150, 64, 1] + ([2000, 2100] if large else [])
    idx = [1, 0, 1, -1, 2, 0] + ([2, 1] if large else [])
    wl = W.fused_custom(lens, idx, H=512, K=32, L=3,
                        slices=[(0, 256), (256, 128), (384, 128)], H_out=520, add=add, seed=33)
    assert (-(-wl.T // 64) >= 64) == large
    df = DeviceFused(wl)
    eager = to_host_bits(df.run())
    assert assert_fused_parity(wl, eager) > 0
    out = df.fresh_out()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        df.run(out)
    for replay in range(4):
        out.copy_(df.out0)                       # eager reset between replays
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host_bits(out), eager), f"replay {replay}"
        other = to_host_bits(df.run())           # eager work in between
        torch.cuda.synchronize()
        assert np.array_equal(other, eager)
