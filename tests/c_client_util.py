"""Files for examples/sgmv_c_client (the plain C-ABI client of libsgmv):
a workload written as the raw arrays and problem line the client reads."""
import os
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "segmented_gather_gemm_amd", "examples", "sgmv_c_client")
DTYPE_CODES = {"f16": 0, "bf16": 1, "f32": 2}


def client_path() -> str:
    if not os.path.exists(CLIENT):
        raise FileNotFoundError(f"{CLIENT} is missing: build it with "
                                "`python -c 'import __graft_entry__ as g; g.build()'`")
    return CLIENT


def run_client(mode: str, d, timeout=120) -> subprocess.CompletedProcess:
    return subprocess.run([client_path(), mode, str(d)], capture_output=True, text=True,
                          timeout=timeout)


def _meta(d, start, lens, idx):
    for name, a in (("start", start), ("lens", lens), ("idx", idx)):
        np.ascontiguousarray(a, dtype=np.int64).tofile(os.path.join(d, f"{name}.bin"))


def write_expand(d, wl):
    """One-slice expand workload -> <d>/problem.txt and the raw arrays."""
    assert len(wl.slices) == 1 and not wl.per_token
    s = wl.slices[0]
    T, H = wl.out0.shape
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write(f"{T} {wl.K} {s.N} {H} {wl.L} {s.offset} {DTYPE_CODES[s.x_dtype]} "
                f"{DTYPE_CODES[s.w_dtype]} {DTYPE_CODES[wl.out_dtype]} {int(wl.add)} "
                f"{wl.batches}\n")
    np.ascontiguousarray(s.x).tofile(os.path.join(d, "x.bin"))
    np.ascontiguousarray(s.w).tofile(os.path.join(d, "w.bin"))
    np.ascontiguousarray(wl.out0).tofile(os.path.join(d, "out0.bin"))
    _meta(d, wl.start, wl.lens, wl.idx)


def write_shrink(d, wl):
    """One-slice shrink workload -> <d>/problem.txt and the raw arrays."""
    assert len(wl.lora_a) == 1
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write(f"{wl.T} {wl.H} {wl.K} {wl.L} {DTYPE_CODES[wl.x_dtype]} "
                f"{DTYPE_CODES[wl.a_dtype]} {DTYPE_CODES[wl.out_dtype]} {float(wl.scale)!r} "
                f"{wl.batches}\n")
    np.ascontiguousarray(wl.x).tofile(os.path.join(d, "x.bin"))
    np.ascontiguousarray(wl.lora_a[0]).tofile(os.path.join(d, "a.bin"))
    np.ascontiguousarray(wl.outs0[0]).tofile(os.path.join(d, "out0.bin"))
    _meta(d, wl.start, wl.lens, wl.idx)


def write_multi(d, wl):
    """Multi-slice expand workload -> <d>/problem.txt and the raw arrays."""
    assert not wl.per_token
    T, H = wl.out0.shape
    s0 = wl.slices[0]
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write(f"{T} {wl.K} {H} {wl.L} {len(wl.slices)} {DTYPE_CODES[s0.x_dtype]} "
                f"{DTYPE_CODES[s0.w_dtype]} {DTYPE_CODES[wl.out_dtype]} {int(wl.add)} "
                f"{wl.batches}\n")
        for s in wl.slices:
            f.write(f"{s.N} {s.offset}\n")
    for i, s in enumerate(wl.slices):
        np.ascontiguousarray(s.x).tofile(os.path.join(d, f"x{i}.bin"))
        np.ascontiguousarray(s.w).tofile(os.path.join(d, f"w{i}.bin"))
    np.ascontiguousarray(wl.out0).tofile(os.path.join(d, "out0.bin"))
    _meta(d, wl.start, wl.lens, wl.idx)


def write_fused(d, wl):
    """Fused shrink-expand workload -> <d>/problem.txt and the raw arrays."""
    T, H_out = wl.out0.shape
    with open(os.path.join(d, "problem.txt"), "w") as f:
        f.write(f"{wl.T} {wl.x.shape[1]} {wl.K} {wl.L} {len(wl.lora_a)} "
                f"{DTYPE_CODES[wl.x_dtype]} {DTYPE_CODES[wl.w_dtype]} "
                f"{DTYPE_CODES[wl.out_dtype]} {int(wl.add)} {len(wl.lens)} "
                f"{float(wl.scale)!r} {H_out}\n")
        for b, off in zip(wl.lora_b, wl.offsets):
            f.write(f"{b.shape[1]} {off}\n")
    np.ascontiguousarray(wl.x).tofile(os.path.join(d, "x.bin"))
    for i, (a, b) in enumerate(zip(wl.lora_a, wl.lora_b)):
        np.ascontiguousarray(a).tofile(os.path.join(d, f"a{i}.bin"))
        np.ascontiguousarray(b).tofile(os.path.join(d, f"b{i}.bin"))
    np.ascontiguousarray(wl.out0).tofile(os.path.join(d, "out0.bin"))
    _meta(d, wl.start, wl.lens, wl.idx)


def read_out(d, shape, dtype: str) -> np.ndarray:
    raw = np.fromfile(os.path.join(d, "out.bin"), dtype=np.float32 if dtype == "f32" else np.uint16)
    return raw.reshape(shape)
