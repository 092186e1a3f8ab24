"""The C-ABI boundary driven by a plain C++ client: examples/sgmv_c_client
loads libsgmv with only the HIP runtime and include/sgmv.h in the process
(no Python, no torch), allocates with hipMalloc, enqueues sgmv_expand_slice,
sgmv_expand_multi_slice, sgmv_shrink or sgmv_fused_shrink_expand (the
descriptor arrays laid out by the header itself) on a stream of its own and
copies the result back.  The problems are seeded workloads written to
files; the results are compared with the oracle as in the other parity
tests."""
import pytest

import sgmv_workloads as W
from c_client_util import (read_out, run_client, write_expand, write_fused, write_multi,
                           write_shrink)
from gpu_util import assert_fused_parity, assert_parity, assert_shrink_parity

pytestmark = pytest.mark.gpu


def _expand_cases():
    return [W.tiny_ref(0), W.WORKLOADS["llama7b_q_proj"](0),
            W.custom([40, 3, 0, 19, 70], [1, 0, 1, -1, 0], K=32, N=256, H=400, off=16, L=2,
                     x_dtype="f32", w_dtype="bf16", out_dtype="bf16", add=True, seed=41,
                     name="custom_f32_add")]


@pytest.mark.parametrize("case", range(3))
def test_c_client_expand_matches_oracle(tmp_path, case):
    wl = _expand_cases()[case]
    print(f"case {wl.name} T={wl.out0.shape[0]} via the C client", flush=True)
    write_expand(tmp_path, wl)
    r = run_client("expand", tmp_path)
    assert r.returncode == 0, r.stderr
    got = read_out(tmp_path, wl.out0.shape, wl.out_dtype)
    assert_parity(wl, got)


def _shrink_case(name):
    if name == "shrink_tiny":
        return W.shrink_tiny(0)
    if name == "balanced":
        # more 64-token units than compute units: parts through the workspace
        import torch
        units = torch.cuda.get_device_properties(0).multi_processor_count + 42
        return W.shrink_custom([64] * units, [i % 5 for i in range(units)], H=512, K=64, L=5,
                               slices=1, x_dtype="bf16", a_dtype="bf16", out_dtype="f32",
                               seed=units)
    return W.SHRINK_WORKLOADS[name](0)


@pytest.mark.parametrize("name", ["shrink_tiny", "shrink_q_proj", "balanced"])
def test_c_client_shrink_matches_oracle(tmp_path, name):
    wl = _shrink_case(name)
    print(f"case {wl.name} T={wl.T} via the C client", flush=True)
    write_shrink(tmp_path, wl)
    r = run_client("shrink", tmp_path)
    assert r.returncode == 0, r.stderr
    got = read_out(tmp_path, wl.outs0[0].shape, wl.out_dtype)
    assert assert_shrink_parity(wl, [got]) > 0


def test_c_client_reports_a_rejected_call(tmp_path):
    """A call the library rejects (slice window past the output's columns)
    comes back as a nonzero exit with sgmv_last_error's text; nothing is
    launched."""
    wl = W.tiny_ref(0)
    write_expand(tmp_path, wl)
    s = wl.slices[0]
    T, H = wl.out0.shape
    with open(tmp_path / "problem.txt", "w") as f:
        f.write(f"{T} {wl.K} {s.N} {H} {wl.L} {H - s.N + 1} 0 0 0 0 {wl.batches}\n")
    r = run_client("expand", tmp_path)
    assert r.returncode == 1
    assert "sgmv_expand_slice returned 1" in r.stderr


@pytest.mark.parametrize("name", ["gqa_qkv", "custom3"])
def test_c_client_multi_slice_matches_oracle(tmp_path, name):
    wl = (W.WORKLOADS["gqa_qkv"](0) if name == "gqa_qkv" else
          W.custom([40, 3, 0, 19, 70], [1, 0, 1, -1, 0], K=32, N=256, H=600, off=16, L=2,
                   add=True, seed=43, extra_slices=[(300, 70), (400, 136)], name="custom3"))
    print(f"case {wl.name} slices={len(wl.slices)} via the C client", flush=True)
    write_multi(tmp_path, wl)
    r = run_client("multi", tmp_path)
    assert r.returncode == 0, r.stderr
    assert_parity(wl, read_out(tmp_path, wl.out0.shape, wl.out_dtype))


@pytest.mark.parametrize("add", [False, True])
def test_c_client_fused_matches_oracle(tmp_path, add):
    wl = W.fused_custom([90, 3, 0, 150, 64, 1], [1, 0, 1, -1, 2, 0], H=512, K=32, L=3,
                        slices=[(0, 256), (256, 128), (384, 128)], H_out=520, add=add, seed=44)
    print(f"case fused add={add} via the C client", flush=True)
    write_fused(tmp_path, wl)
    r = run_client("fused", tmp_path)
    assert r.returncode == 0, r.stderr
    assert assert_fused_parity(wl, read_out(tmp_path, wl.out0.shape, wl.out_dtype)) > 0
