"""Helpers for the GPU parity tests: move a seeded workload to the device,
run libsgmv through its Python binding (the C ABI), bring the output back as
bits, and compare with the CPU oracle."""
import numpy as np

import oracle

# |gpu - ref| <= atol + rtol * |ref| per output dtype, ref = exact fp64 value.
TOLERANCE = {"bf16": (1e-3, 8e-3), "f16": (1e-3, 2e-3), "f32": (1e-5, 1e-5)}


def torch_dtype(name):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[name]


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    from sgmv_workloads import to_torch
    return to_torch(a, dtype, device)


def to_host_bits(t) -> np.ndarray:
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


class DeviceWorkload:
    """A workload's tensors on the GPU."""

    def __init__(self, wl, device="cuda", meta_dtype=None):
        import torch
        self.wl = wl
        md = meta_dtype or torch.int64
        self.start = torch.from_numpy(wl.start).to(device=device, dtype=md)
        self.lens = torch.from_numpy(wl.lens).to(device=device, dtype=md)
        self.idx = torch.from_numpy(wl.idx).to(device=device, dtype=md)
        self.x = [to_device(s.x, s.x_dtype, device) for s in wl.slices]
        self.w = [to_device(np.ascontiguousarray(s.w).reshape(s.w.shape[0], -1), s.w_dtype,
                            device).view(s.w.shape) for s in wl.slices]
        self.out0 = to_device(wl.out0, wl.out_dtype, device)

    def fresh_out(self):
        return self.out0.clone() if self.out0.is_contiguous() else self._strided_clone()

    def _strided_clone(self):
        import torch
        full = torch.empty((self.out0.shape[0], self.out0.stride(0)), dtype=self.out0.dtype,
                           device=self.out0.device)
        full[:, :self.out0.shape[1]] = self.out0
        full[:, self.out0.shape[1]:] = 0
        return full[:, :self.out0.shape[1]]

    def run_single(self, out, slice_index=0, max_seq_length=None, batches=None):
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        s = wl.slices[slice_index]
        sg.sgmv_expand_slice(self.x[slice_index], self.w[slice_index], out, self.start,
                             self.lens, self.idx, wl.batches if batches is None else batches,
                             wl.max_seq_len if max_seq_length is None else max_seq_length,
                             s.offset, s.N, wl.add)
        return out

    def run_all_single(self, out):
        for i in range(len(self.wl.slices)):
            self.run_single(out, i)
        return out

    def run_bgmv(self, out):
        """The per-token entry point (the workload's segments must be rows)."""
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        s = wl.slices[0]
        sg.bgmv_expand_slice(self.x[0], self.w[0], out, self.idx, s.offset, s.N, wl.add)
        return out

    def run_multi(self, out):
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        sg.sgmv_expand_multi_slice([(self.x[i], self.w[i], s.offset)
                                    for i, s in enumerate(wl.slices)], out, self.start,
                                   self.lens, self.idx, wl.batches, wl.max_seq_len, wl.add)
        return out


def oracle_check(wl, cand_bits, rows=None, threads=0):
    atol, rtol = TOLERANCE[wl.out_dtype]
    slices = [oracle.Slice(s.x, s.x_dtype, s.w, s.w_dtype, s.offset) for s in wl.slices]
    return oracle.check(slices, np.ascontiguousarray(wl.out0), np.ascontiguousarray(cand_bits),
                        wl.out_dtype, wl.start, wl.lens, wl.idx,
                        wl.add, wl.K, wl.L, atol, rtol, rows=rows, threads=threads)


def assert_parity(wl, cand_bits, rows=None):
    rep = oracle_check(wl, cand_bits, rows=rows)
    assert rep.ok, (f"{wl.name}: {rep.bad_values} bad values, {rep.bad_untouched} changed "
                    f"untouched elements, first at {rep.first_bad}, max |err| "
                    f"{rep.max_abs_err:.3g}, worst err/tol {rep.max_tol_ratio:.3g}")
    assert rep.checked_values > 0 or not wl.active_mask().any()
    return rep


# --------------------------------------------------------------------------
# LoRA-A projection (shrink).
# --------------------------------------------------------------------------

def _device_clone(t):
    """Clone keeping a strided view's row stride (padding zeroed)."""
    import torch
    if t.is_contiguous():
        return t.clone()
    full = torch.zeros((t.shape[0], t.stride(0)), dtype=t.dtype, device=t.device)
    full[:, :t.shape[1]] = t
    return full[:, :t.shape[1]]


class DeviceShrink:
    """A shrink workload's tensors on the GPU."""

    def __init__(self, wl, device="cuda"):
        import torch
        self.wl = wl
        self.start = torch.from_numpy(wl.start).to(device)
        self.lens = torch.from_numpy(wl.lens).to(device)
        self.idx = torch.from_numpy(wl.idx).to(device)
        self.x = to_device(wl.x, wl.x_dtype, device)
        self.a = [to_device(np.ascontiguousarray(a).reshape(a.shape[0], -1), wl.a_dtype,
                            device).view(a.shape) for a in wl.lora_a]
        self.outs0 = [to_device(o, wl.out_dtype, device) for o in wl.outs0]

    def fresh_outs(self):
        return [_device_clone(o) for o in self.outs0]

    def run(self, outs=None, multi=True, idx=None, workspace=True):
        """One multi-slice call, or one sgmv_shrink call per slice (`workspace`
        as the binding takes it: True = the device's shared buffer)."""
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        outs = self.fresh_outs() if outs is None else outs
        idx = self.idx if idx is None else idx
        if multi:
            sg.sgmv_shrink_multi_slice(self.x, list(zip(self.a, outs)), self.start, self.lens,
                                       idx, wl.batches, wl.max_seq_len, wl.scale, workspace)
        else:
            for a, o in zip(self.a, outs):
                sg.sgmv_shrink(self.x, a, o, self.start, self.lens, idx, wl.batches,
                               wl.max_seq_len, wl.scale, workspace)
        return outs


# Unit roundoff of fp32, the accumulation type.
U_FP32 = 2.0 ** -24


def shrink_abs_dot(wl, si, rows, ra):
    """sum_h |x[t][h] * A[a][k][h]| for the given rows (numpy, from the stored
    values; float32 inputs cast to the weight dtype as the products see them)."""
    from oracle_pins_util import np_cast_input, np_values
    x = np_cast_input(np.ascontiguousarray(wl.x[rows]), wl.x_dtype, wl.a_dtype)
    av = np.abs(np_values(wl.lora_a[si], wl.a_dtype))
    out = np.zeros((len(rows), wl.K))
    for a in np.unique(ra[rows]):
        m = ra[rows] == a
        out[m] = np.abs(x[m]) @ av[a].T
    return out


def shrink_sum_depth(wl):
    """The most fp32 roundings an exact 16-bit product can pass through on
    its way into a result of the kernel the library picks for this shrink
    workload.  The register-tiled (MFMA) kernels -- taken, as at the ABI,
    when rank and hidden are multiples of 8, every row stride is a multiple
    of 16 bytes and one adapter's lora_A rows span less than 2 GiB (the test
    buffers are 16-byte aligned) -- add a product into at most 32 others
    inside one 32-wide MFMA step, then once per later step (ceil(H / 32)),
    then at most 3 times where the split-H waves or the balanced split-T
    parts are added (8 allowed): 32 + ceil(H / 32) + 8.  The generic kernel
    accumulates the H products one after the other: H."""
    x_ok = wl.x.strides[0] % 16 == 0 and all(o.strides[0] % 16 == 0 for o in wl.outs0)
    p = 1
    while p < (wl.K + 15) // 16:
        p *= 2
    fast = (wl.K % 8 == 0 and wl.H % 8 == 0 and x_ok and 32 * p * wl.H < 2 ** 31)
    return min(wl.H, 32 + -(-wl.H // 32) + 8) if fast else wl.H


def assert_shrink_parity(wl, cand_bits, rows=None, idx=None, exact=False, depth=None):
    """GPU outputs (one bits array per slice) vs the oracle: every computed
    value of an active row within tolerance of the exact value (non-finite
    exactly where the rounded exact value is), every other row bit-identical
    to the prior output.  ``rows`` samples the rows whose values are checked
    (the untouched check always covers every row).  ``exact``: the bits must
    equal the oracle's (integer data, where every fp32 partial sum is exact).

    Tolerance: the output dtype's atol + rtol * |ref| (which covers the final
    rounding and the scale's rounding), plus the bound on fp32 summation of
    the H exact 16-bit products, gamma_d * |scale| * sum_h |x_h a_h| with
    gamma_d = d u / (1 - d u), u = 2^-24 and d the most roundings any
    product passes through (shrink_sum_depth: 32 + ceil(H / 32) + 8 on the
    MFMA kernels, H on the generic one; the recursive summation bound, which
    holds for every order and grouping within that depth; ``depth`` overrides
    it for buffers other than the workload's own).
    Returns the number of values checked."""
    atol, rtol = TOLERANCE[wl.out_dtype]
    depth = shrink_sum_depth(wl) if depth is None else depth
    gamma = depth * U_FP32 / (1.0 - depth * U_FP32)
    idx = wl.idx if idx is None else idx
    outs = [o.copy() for o in wl.outs0]
    refs = oracle.shrink(wl.x, wl.x_dtype, wl.lora_a, wl.a_dtype, outs, wl.out_dtype, wl.start,
                         wl.lens, idx, wl.scale, rows=rows, want_ref=True)
    active = np.zeros(wl.T, dtype=bool)
    for s, n, a in zip(wl.start, wl.lens, idx):
        if 0 <= a < wl.L and n > 0:
            active[s:s + n] = True
    checked = np.zeros(wl.T, dtype=bool)
    checked[np.arange(wl.T) if rows is None else np.asarray(rows)] = True
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, idx):
        if 0 <= a < wl.L and n > 0:
            ra[s:s + n] = a
    from oracle_pins_util import np_values
    n_checked = 0
    for si, (cand, ref, rounded) in enumerate(zip(cand_bits, refs, outs)):
        assert np.array_equal(cand[~active], wl.outs0[si][~active]), \
            f"{wl.name} slice {si}: rows without an adapter changed"
        m = active & checked
        if exact:
            assert np.array_equal(cand[m], rounded[m]), f"{wl.name} slice {si}: bits differ"
            n_checked += int(m.sum()) * wl.K
            continue
        got = np_values(np.ascontiguousarray(cand[m]), wl.out_dtype)
        exp = ref[m]
        exp_rounded = np_values(np.ascontiguousarray(rounded[m]), wl.out_dtype)
        finite = np.isfinite(exp_rounded)
        assert np.array_equal(np.isfinite(got), finite), f"{wl.name} slice {si}: non-finite mismatch"
        err = np.abs(got[finite] - exp[finite])
        acc = gamma * abs(wl.scale) * shrink_abs_dot(wl, si, np.nonzero(m)[0], ra)
        tol = atol + rtol * np.abs(exp[finite]) + acc[finite]
        bad = np.nonzero(err > tol)[0]
        assert bad.size == 0, (f"{wl.name} slice {si}: {bad.size} values out of tolerance, worst "
                               f"err/tol {float(np.max(err / tol)):.3g}")
        n_checked += int(m.sum()) * wl.K
    return n_checked


# --------------------------------------------------------------------------
# Fused LoRA delta (shrink and expand in one call).
# --------------------------------------------------------------------------

class DeviceFused:
    """A fused workload's tensors on the GPU."""

    def __init__(self, wl, device="cuda"):
        import torch
        self.wl = wl
        self.start = torch.from_numpy(wl.start).to(device)
        self.lens = torch.from_numpy(wl.lens).to(device)
        self.idx = torch.from_numpy(wl.idx).to(device)
        self.x = to_device(wl.x, wl.x_dtype, device)
        self.a = [to_device(np.ascontiguousarray(a).reshape(a.shape[0], -1), wl.w_dtype,
                            device).view(a.shape) for a in wl.lora_a]
        self.b = [to_device(np.ascontiguousarray(b).reshape(b.shape[0], -1), wl.w_dtype,
                            device).view(b.shape) for b in wl.lora_b]
        self.out0 = to_device(wl.out0, wl.out_dtype, device)

    def fresh_out(self):
        return _device_clone(self.out0)

    def run(self, out=None):
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        out = self.fresh_out() if out is None else out
        sg.sgmv_fused_shrink_expand(self.x, list(zip(self.a, self.b, wl.offsets)), out,
                                    self.start, self.lens, self.idx, wl.batches,
                                    wl.max_seq_len, wl.scale, wl.add)
        return out

    def run_two(self, out=None, workspace=None):
        """The two-call path: sgmv_shrink_multi_slice into weight-dtype
        projections, then sgmv_expand_multi_slice of them.  Without a
        workspace (the default here) the shrink sums every hidden step in one
        accumulator, as the fused kernel does, so the two paths agree bit for
        bit; with one, large batches add hidden parts in another order."""
        import torch
        import segmented_gather_gemm_amd as sg
        wl = self.wl
        out = self.fresh_out() if out is None else out
        ys = [torch.zeros((wl.T, wl.K), dtype=torch_dtype(wl.w_dtype), device=out.device)
              for _ in wl.lora_a]
        sg.sgmv_shrink_multi_slice(self.x, list(zip(self.a, ys)), self.start, self.lens,
                                   self.idx, wl.batches, wl.max_seq_len, wl.scale, workspace)
        sg.sgmv_expand_multi_slice([(y, b, off) for y, b, off in zip(ys, self.b, wl.offsets)],
                                   out, self.start, self.lens, self.idx, wl.batches,
                                   wl.max_seq_len, wl.add)
        return ys, out


def fused_written_mask(wl):
    rows = np.zeros(wl.T, dtype=bool)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if 0 <= a < wl.L and n > 0:
            rows[s:s + n] = True
    cols = np.zeros(wl.out0.shape[1], dtype=bool)
    for off, b in zip(wl.offsets, wl.lora_b):
        cols[off:off + b.shape[1]] = True
    return rows, cols


def assert_fused_parity(wl, cand_bits, exact=False):
    """GPU output of a fused call vs oracle.fused: elements outside (active
    rows x windows) keep their bits; with ``exact`` every bit equals the
    oracle's (integer data); otherwise each written value is within

        atol + rtol |R| + sum_k delta_k |B[a][n][k]|,
        delta_k = ulp_w(2 (|y_k| + e_k)) + e_k,
        e_k = |scale| (gamma_d + 2^-23) sum_h |x_h A[a][k][h]|,

    of the exact expand R of the oracle's projection y: the GPU's fp32
    projection differs from the exact one by at most e_k (summation of H
    exact products in any order and grouping in which no product meets more
    than d = 32 + ceil(H / 32) + 8 roundings -- the fused kernel runs the
    split-T or split-H MFMA contraction, see shrink_sum_depth -- then the
    scale's rounding), so its
    rounding to the weight dtype can land at most delta_k from the oracle's;
    atol and rtol cover the expand's own fp32 sums and final rounding.
    Returns the number of values compared."""
    from oracle_pins_util import np_cast_input, np_values, ulp
    out = wl.out0.copy()
    ys, refs = oracle.fused(wl.x, wl.x_dtype, wl.lora_a, wl.lora_b, wl.w_dtype, wl.offsets, out,
                            wl.out_dtype, wl.start, wl.lens, wl.idx, wl.scale, wl.add,
                            want_ref=True)
    rows, cols = fused_written_mask(wl)
    bits = cand_bits.view(np.uint32) if wl.out_dtype == "f32" else cand_bits
    prior = wl.out0.view(np.uint32) if wl.out_dtype == "f32" else wl.out0
    untouched = ~(rows[:, None] & cols[None, :])
    assert np.array_equal(bits[untouched], prior[untouched]), \
        f"{wl.name}: elements outside the written region changed"
    if exact:
        ob = out.view(np.uint32) if wl.out_dtype == "f32" else out
        assert np.array_equal(bits, ob), f"{wl.name}: bits differ from the oracle"
        return int(rows.sum() * cols.sum())
    atol, rtol = TOLERANCE[wl.out_dtype]
    depth = min(wl.H, 32 + -(-wl.H // 32) + 8)
    gamma = depth * U_FP32 / (1.0 - depth * U_FP32) + 2.0 ** -23
    x = np.abs(np_cast_input(np.ascontiguousarray(wl.x), wl.x_dtype, wl.w_dtype))
    ra = np.full(wl.T, -1, dtype=np.int64)
    for s, n, a in zip(wl.start, wl.lens, wl.idx):
        if 0 <= a < wl.L and n > 0:
            ra[s:s + n] = a
    act = np.nonzero(rows)[0]
    n_checked = 0
    for y, a_s, b_s, off, ref in zip(ys, wl.lora_a, wl.lora_b, wl.offsets, refs):
        N = b_s.shape[1]
        av = np.abs(np_values(a_s, wl.w_dtype))
        bv = np.abs(np_values(b_s, wl.w_dtype))
        yv = np.abs(np_values(y, wl.w_dtype))
        extra = np.zeros((wl.T, N))
        for a in np.unique(ra[act]):
            m = ra == a
            e = abs(wl.scale) * gamma * (x[m] @ av[a].T)
            delta = ulp(2.0 * (yv[m] + e), wl.w_dtype) + e
            extra[m] = delta @ bv[a].T
        got = np_values(np.ascontiguousarray(cand_bits[act][:, off:off + N]), wl.out_dtype)
        exp = ref[act]
        assert np.isfinite(got).all(), f"{wl.name}: non-finite values"
        err = np.abs(got - exp)
        tol = atol + rtol * np.abs(exp) + extra[act]
        bad = np.argwhere(err > tol)
        assert bad.size == 0, (f"{wl.name}: {len(bad)} values out of tolerance, first at "
                               f"{tuple(bad[0])}, worst err/tol {float(np.max(err / tol)):.3g}")
        n_checked += err.size
    return n_checked
