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
