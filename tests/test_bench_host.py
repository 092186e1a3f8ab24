"""Host-side parts of the benchmark: the byte model against a hand count,
the source hash, and the refusal of a multi-GPU run (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

import bench
import sgmv_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_byte_model_hand_count():
    # 3 segments: 5 rows adapter 1, 7 rows index -1, 2 rows adapter 1; rank 16,
    # slice 64 of bf16, accumulate: active rows 7, one distinct adapter.
    wl = W.custom([5, 7, 2], [1, -1, 1], K=16, N=64, H=80, off=8, L=2, add=True)
    total, t_act, distinct = bench.byte_model(wl)
    assert (t_act, distinct) == (7, 1)
    assert total == 7 * 16 * 2 + 1 * 64 * 16 * 2 + 7 * 64 * 2 * 2


def test_byte_model_multi_slice_and_fp32_input():
    wl = W.custom([4, 4], [0, 1], K=8, N=16, H=64, off=0, L=2, x_dtype="f32", add=False,
                  extra_slices=[(32, 8)])
    total, t_act, distinct = bench.byte_model(wl)
    per_slice = lambda n: 8 * 8 * 4 + 2 * n * 8 * 2 + 8 * n * 2
    assert total == per_slice(16) + per_slice(8)


def test_named_workload_byte_counts():
    total, t_act, distinct = bench.byte_model(W.llama7b_q_proj(0))
    assert (t_act, distinct) == (1279, 3)
    assert total == 1279 * 16 * 2 + 3 * 4096 * 16 * 2 + 1279 * 4096 * 2 * 2


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16
    # the shrink's hash also covers its own sources
    assert bench.kernel_source_hash("shrink") != bench.kernel_source_hash("expand")


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_reports_multi_and_single_core_rates():
    import bench
    import sgmv_workloads as W
    wl = W.tiny_ref(0)
    mb, _, _ = bench.byte_model(wl)
    cpu = bench.cpu_baseline(wl, mb, 0.05)
    assert cpu["kind"] == "oracle" and cpu["unit"] == "GB/s"
    assert cpu["value"] > 0 and cpu["single_core_gbs"] > 0 and cpu["reps"] >= 1
    assert cpu["cores"] >= 1 and "tiny_ref" in cpu["sample"]


def test_shrink_byte_model_hand_count():
    # segments: 5 rows adapter 1, 7 rows index -1, 2 rows adapter 0; hidden 64
    # bf16 -> rank 16, two slices, float32 output: 7 active rows, 2 adapters.
    wl = W.shrink_custom([5, 7, 2], [1, -1, 0], H=64, K=16, L=2, slices=2, out_dtype="f32")
    total, t_act, distinct = bench.shrink_byte_model(wl)
    assert (t_act, distinct) == (7, 2)
    assert total == 7 * 64 * 2 + 2 * 2 * 16 * 64 * 2 + 2 * 7 * 16 * 4


def test_shrink_named_workload_byte_counts():
    total, t_act, distinct = bench.shrink_byte_model(W.shrink_q_proj(0))
    assert (t_act, distinct) == (1279, 3)
    assert total == 1279 * 4096 * 2 + 3 * 16 * 4096 * 2 + 1279 * 16 * 2


def test_shrink_cpu_baseline():
    wl = W.shrink_tiny(0)
    cpu = bench.shrink_cpu_baseline(wl, 0.05)
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["single_core_gbs"] > 0
    assert "shrink_tiny" in cpu["sample"]


def test_fused_byte_model_hand_count():
    # segments: 5 rows adapter 1, 7 rows index -1, 2 rows adapter 0; hidden 64
    # bf16 -> rank 16 -> slices of 32 and 16 columns, bf16 output, accumulate:
    # 7 active rows, 2 adapters; the projection never leaves the chip.
    wl = W.fused_custom([5, 7, 2], [1, -1, 0], H=64, K=16, L=2, slices=[(0, 32), (32, 16)],
                        H_out=48, add=True)
    total, read, t_act, distinct = bench.fused_byte_model(wl)
    assert (t_act, distinct) == (7, 2)
    want_read = 7 * 64 * 2 + 2 * 2 * 16 * 64 * 2 + 2 * 48 * 16 * 2 + 7 * 48 * 2
    assert read == want_read and total == want_read + 7 * 48 * 2


def test_small_fused_workloads_follow_their_recipes():
    # fused_q_proj: llama7b_q_proj's segments and indices, one 4096-wide slice
    q, base = W.fused_q_proj(0), W.llama7b_q_proj(0)
    assert np.array_equal(q.lens, base.lens) and np.array_equal(q.idx, base.idx)
    assert (q.H, q.K, q.L, q.add, q.offsets) == (4096, 16, 4, True, [0])
    assert [b.shape for b in q.lora_b] == [(4, 4096, 16)]
    # fused_decode_qkv: 256 one-token segments in order, indices in -1..31
    d = W.fused_decode_qkv(0)
    assert d.batches == 256 and (d.lens == 1).all()
    assert np.array_equal(d.start, np.arange(256))
    assert d.idx.min() >= -1 and d.idx.max() <= 31 and (d.idx == -1).any()
    assert d.offsets == [o for o, _ in W.QKV_SLICES]
    # both stay below 64 units of 64 tokens (the fused call's 16-row form)
    for wl in (q, d):
        assert -(-wl.T // 64) < 64
