"""GPU parity of the per-token (BGMV) entry point, sgmv_bgmv_expand_slice:
every token takes its own adapter (the counterpart the page's Description
names), checked against the CPU oracle with row t as segment t, and
bit-identical to sgmv_expand_slice over the same one-row segments."""
import numpy as np
import pytest

import sgmv_workloads as W
from gpu_util import DeviceWorkload, assert_parity, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,K,N,dts,add", [
    (1, 16, 256, ("bf16", "bf16", "bf16"), True),
    (7, 8, 200, ("f16", "f16", "f16"), False),
    (64, 32, 1024, ("bf16", "bf16", "f32"), True),
    (300, 64, 512, ("f32", "bf16", "bf16"), False),
    (512, 128, 768, ("f16", "f16", "f16"), True),
    (513, 16, 256, ("bf16", "bf16", "bf16"), True),
    (2000, 16, 512, ("bf16", "bf16", "bf16"), False),
    (4000, 8, 128, ("f16", "f16", "f16"), True),
    (90, 7, 96, ("f16", "f16", "f32"), True),        # rank 7: the generic kernel
])
def test_bgmv_parity(T, K, N, dts, add):
    x_dt, w_dt, o_dt = dts
    rng = np.random.default_rng(T + K)
    L = 24
    idx = rng.integers(-1, L, size=T)
    wl = W.per_token(idx.tolist(), K=K, N=N, H=N + 64, off=32, L=L, x_dtype=x_dt, w_dtype=w_dt,
                     out_dtype=o_dt, add=add, seed=T)
    dw = DeviceWorkload(wl)
    out = dw.run_bgmv(dw.fresh_out())
    assert_parity(wl, to_host_bits(out))


def test_bgmv_equals_sgmv_with_one_row_segments():
    rng = np.random.default_rng(5)
    idx = rng.integers(-1, 6, size=100)
    wl = W.per_token(idx.tolist(), K=32, N=512, H=512, off=0, L=6, add=True, seed=5)
    dw = DeviceWorkload(wl)
    a = to_host_bits(dw.run_bgmv(dw.fresh_out()))
    b = to_host_bits(dw.run_single(dw.fresh_out()))
    assert np.array_equal(a, b)


def test_bgmv_decode_workload():
    wl = W.bgmv_decode(0)
    dw = DeviceWorkload(wl)
    out = dw.run_bgmv(dw.fresh_out())
    assert_parity(wl, to_host_bits(out))


def test_bgmv_all_tokens_without_adapter_touch_nothing():
    wl = W.per_token([-1] * 40, K=16, N=256, H=256, off=0, L=3, add=False, seed=6)
    dw = DeviceWorkload(wl)
    out = to_host_bits(dw.run_bgmv(dw.fresh_out()))
    assert np.array_equal(out, wl.out0)


@pytest.mark.parametrize("T,L", [(256, 1023), (300, 1024), (300, 1025), (400, 1200), (512, 2),
                                 (3000, 7)])
def test_bgmv_adapter_order_few_and_many_adapters(T, L):
    # Up to 1024 adapters the tokens of each adapter are gathered into row
    # tiles (a table of adapter buckets), past that each token is its own
    # tile; from two adapters (long runs) to more adapters than tokens.
    rng = np.random.default_rng(T + L)
    idx = rng.integers(-1, L, size=T)
    wl = W.per_token(idx.tolist(), K=16, N=256, H=256, off=0, L=L, add=True, seed=T)
    dw = DeviceWorkload(wl)
    out = dw.run_bgmv(dw.fresh_out())
    assert_parity(wl, to_host_bits(out))
