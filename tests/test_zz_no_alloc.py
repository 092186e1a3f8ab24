"""The allocation-free shrink entry point, sgmv_shrink_multi_slice_noalloc,
called through the C ABI: its workspace is the library's static device array
(one per device), cleared of part counters at every call.  Two calls in a
row, the second with a smaller batch, each compared bit for bit with
sgmv_shrink_multi_slice on a workspace of the caller's (the same kernels,
so the same bits) and with the oracle."""
import ctypes

import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceShrink, assert_shrink_parity, to_host_bits

pytestmark = pytest.mark.gpu


def noalloc_call(dw, outs):
    """One sgmv_shrink_multi_slice_noalloc call through the C ABI (ctypes)."""
    import segmented_gather_gemm_amd as sg
    import torch
    wl = dw.wl
    arr = (sg.ShrinkSliceDesc * len(outs))()
    for i, (a, o) in enumerate(zip(dw.a, outs)):
        arr[i] = sg.ShrinkSliceDesc(sg._stack_a(a, "a"), sg._matrix(o, "out"))
    stream = torch.cuda.current_stream().cuda_stream
    st = sg.lib.sgmv_shrink_multi_slice_noalloc(
        sg._matrix(dw.x, "x"), arr, len(outs), dw.start.data_ptr(), dw.lens.data_ptr(),
        dw.idx.data_ptr(), wl.batches, wl.max_seq_len, ctypes.c_float(wl.scale), stream)
    assert st == sg.SGMV_OK, sg.lib.sgmv_last_error().decode()
    return outs


def test_noalloc_shrink_equals_the_workspace_call_twice_in_a_row():
    import torch
    import segmented_gather_gemm_amd as sg
    C = torch.cuda.get_device_properties(0).multi_processor_count
    # first: a balanced batch (C + 42 units of 64 tokens, parts through the
    # static array); second: a smaller balanced batch (C + 5 units)
    big = W.shrink_custom([64] * (C + 42), [i % 5 for i in range(C + 42)], H=1024, K=64, L=5,
                          slices=2, x_dtype="bf16", a_dtype="bf16", out_dtype="f32", seed=71)
    small = W.shrink_custom([64] * (C + 5), [i % 3 for i in range(C + 5)], H=512, K=32, L=3,
                            slices=3, x_dtype="f16", a_dtype="f16", out_dtype="bf16", seed=72)
    for wl in (big, small):
        print(f"case {wl.name} T={wl.T} H={wl.H} K={wl.K} slices={len(wl.lora_a)}", flush=True)
        dw = DeviceShrink(wl)
        got = [to_host_bits(o) for o in noalloc_call(dw, dw.fresh_outs())]
        ws = torch.zeros(sg.shrink_workspace_bytes(), dtype=torch.uint8, device="cuda")
        ref = [to_host_bits(o) for o in dw.run(workspace=ws)]
        for g, r in zip(got, ref):
            assert np.array_equal(g, r)
        assert assert_shrink_parity(wl, got) > 0
