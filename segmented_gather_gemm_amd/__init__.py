"""Python binding of libsgmv: SGMV expand-slice on MI355X (gfx950).

Argument marshalling only.  Every step of the operation runs in the HIP
kernels of ``libsgmv.so`` (built in-tree by ``build.py``); PyTorch supplies
device memory and the current stream.  There is no CPU or PyTorch fallback:
if the library is missing, importing this package raises.

Names and argument order follow the wiki page "Implementation: Predibase
Lorax SGMV Expand Slice Kernel" (Signature; I/O Contract):

    sgmv_expand_slice(inputs, lora_b_weights, output_tensor, b_seq_start_loc,
                      seq_len_tensor, lora_indices_tensor, batches,
                      max_seq_length, slice_offset, slice_size, add_inputs=False)

plus the LoRA-A projection that produces those inputs (sgmv_shrink), the
per-token and multi-slice forms, and the two steps fused in one launch
(sgmv_fused_shrink_expand).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "libsgmv.so")

SGMV_OK, SGMV_ERR_INVALID_ARGUMENT, SGMV_ERR_UNSUPPORTED, SGMV_ERR_HIP = range(4)
MAX_SLICES = 8
MAX_FUSED_SLICES = 3

# Every symbol include/sgmv.h declares.
EXPORTED_SYMBOLS = ("sgmv_expand_slice", "sgmv_expand_multi_slice", "sgmv_bgmv_expand_slice",
                    "sgmv_shrink", "sgmv_shrink_multi_slice", "sgmv_shrink_workspace_bytes",
                    "sgmv_shrink_multi_slice_noalloc",
                    "sgmv_fused_shrink_expand", "sgmv_last_error", "sgmv_abi_version")


class Matrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class Stack(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("num", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class SliceDesc(ctypes.Structure):
    _fields_ = [("inputs", Matrix), ("lora_b", Stack), ("slice_offset", ctypes.c_int64),
                ("slice_size", ctypes.c_int64)]


class ShrinkSliceDesc(ctypes.Structure):
    _fields_ = [("lora_a", Stack), ("out", Matrix)]


class FusedSliceDesc(ctypes.Structure):
    _fields_ = [("lora_a", Stack), ("lora_b", Stack), ("slice_offset", ctypes.c_int64)]


def _hip_runtimes_mapped():
    """Distinct HIP runtime files mapped into this process."""
    found = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                path = line.split()[-1] if line.strip() else ""
                if "libamdhip64.so" in os.path.basename(path):
                    found.add(os.path.realpath(path))
    except OSError:
        pass
    return found


def _load_library() -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime.  Load it first so that libsgmv's
    # dependency on libamdhip64.so.7 resolves to that same, already mapped
    # runtime: two HIP runtimes in one process do not share devices, streams
    # or allocations.
    import torch  # noqa: F401
    if not os.path.exists(LIBRARY_PATH):
        raise ImportError(
            f"{LIBRARY_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
            f"g.build()'` (or python segmented_gather_gemm_amd/build.py). There is no fallback.")
    lib = ctypes.CDLL(LIBRARY_PATH)
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    i64, p = ctypes.c_int64, ctypes.c_void_p
    lib.sgmv_expand_slice.argtypes = [Matrix, Stack, Matrix, p, p, p, i64, i64, i64, i64,
                                      ctypes.c_int, p]
    lib.sgmv_expand_slice.restype = ctypes.c_int
    lib.sgmv_expand_multi_slice.argtypes = [ctypes.POINTER(SliceDesc), ctypes.c_int, Matrix, p, p,
                                            p, i64, i64, ctypes.c_int, p]
    lib.sgmv_expand_multi_slice.restype = ctypes.c_int
    lib.sgmv_bgmv_expand_slice.argtypes = [Matrix, Stack, Matrix, p, i64, i64, ctypes.c_int, p]
    lib.sgmv_bgmv_expand_slice.restype = ctypes.c_int
    lib.sgmv_shrink.argtypes = [Matrix, Stack, Matrix, p, p, p, i64, i64, ctypes.c_float, p,
                                ctypes.c_size_t, p]
    lib.sgmv_shrink.restype = ctypes.c_int
    lib.sgmv_shrink_multi_slice.argtypes = [Matrix, ctypes.POINTER(ShrinkSliceDesc), ctypes.c_int,
                                            p, p, p, i64, i64, ctypes.c_float, p,
                                            ctypes.c_size_t, p]
    lib.sgmv_shrink_multi_slice.restype = ctypes.c_int
    lib.sgmv_shrink_workspace_bytes.argtypes = [ctypes.POINTER(ctypes.c_size_t)]
    lib.sgmv_shrink_workspace_bytes.restype = ctypes.c_int
    lib.sgmv_shrink_multi_slice_noalloc.argtypes = [Matrix, ctypes.POINTER(ShrinkSliceDesc),
                                                    ctypes.c_int, p, p, p, i64, i64,
                                                    ctypes.c_float, p]
    lib.sgmv_shrink_multi_slice_noalloc.restype = ctypes.c_int
    lib.sgmv_fused_shrink_expand.argtypes = [Matrix, ctypes.POINTER(FusedSliceDesc), ctypes.c_int,
                                             Matrix, p, p, p, i64, i64, ctypes.c_float,
                                             ctypes.c_int, p]
    lib.sgmv_fused_shrink_expand.restype = ctypes.c_int
    lib.sgmv_last_error.argtypes = []
    lib.sgmv_last_error.restype = ctypes.c_char_p
    lib.sgmv_abi_version.argtypes = []
    lib.sgmv_abi_version.restype = ctypes.c_int
    return lib


lib = _load_library()

import torch as _torch  # noqa: E402  (loaded by _load_library before the library)

_DTYPE_CODES = {_torch.float16: 0, _torch.bfloat16: 1, _torch.float32: 2}
# The current stream's raw handle without building a Stream object (a
# measurable part of a call's host time); the public route where absent.
_RAW_STREAM = getattr(_torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _RAW_STREAM is not None:
        return _RAW_STREAM(device.index)
    return _torch.cuda.current_stream(device).cuda_stream


def _call_on(device, fn, *args):
    """fn(*args) with `device` current (made current only when it is not)."""
    if _torch.cuda.current_device() == device.index:
        return fn(*args)
    with _torch.cuda.device(device):
        return fn(*args)


class SgmvError(RuntimeError):
    """A HIP runtime failure reported by libsgmv."""


def _raise(status: int):
    msg = lib.sgmv_last_error().decode(errors="replace")
    if status == SGMV_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    if status == SGMV_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise SgmvError(msg)


def _dtype_code(t) -> int:
    code = _DTYPE_CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _matrix(t, what: str) -> Matrix:
    shape = t.shape
    if len(shape) != 2:
        raise ValueError(f"{what} must be 2-D, got shape {tuple(shape)}")
    rows, cols = shape
    s0, s1 = t.stride()
    if cols > 1 and s1 != 1:
        raise ValueError(f"{what} must have unit column stride")
    return Matrix(t.data_ptr(), _dtype_code(t), rows, cols, s0 if rows > 1 else max(cols, s0))


def _stack(w, what: str) -> Stack:
    if w.dim() == 4:
        if w.shape[1] != 1:
            raise ValueError(f"{what}: a 4-D lora_b must be (lora_num, 1, slice_size, rank)")
        w = w.squeeze(1)
    shape = w.shape
    if len(shape) != 3:
        raise ValueError(f"{what} must be (lora_num, slice_size, rank), got {tuple(shape)}")
    if not w.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return Stack(w.data_ptr(), _dtype_code(w), shape[0], shape[1], shape[2])


def _meta(t, what: str, device):
    if t.dim() != 1:
        raise ValueError(f"{what} must be 1-D")
    if t.device != device:
        raise ValueError(f"{what} must be on {device}")
    if t.dtype is not _torch.int64 or not t.is_contiguous():
        t = t.to(_torch.int64).contiguous()   # documented marshalling copy
    return t


def _common(output_tensor, metas):
    device = output_tensor.device
    if device.type != "cuda":
        raise ValueError("output_tensor must be a GPU tensor")
    kept = [_meta(m, n, device) for m, n in metas]
    return device, kept


def sgmv_expand_slice(inputs, lora_b_weights, output_tensor, b_seq_start_loc, seq_len_tensor,
                      lora_indices_tensor, batches: int, max_seq_length: int, slice_offset: int,
                      slice_size: int, add_inputs: bool = False):
    """In place: output_tensor[start_b + m, slice_offset:slice_offset + slice_size]
    (+)= inputs[start_b + m] @ lora_b_weights[lora_indices[b]].T for every
    segment b with index != -1.  Enqueued on the current stream."""
    device, (start, lens, idx) = _common(output_tensor, [
        (b_seq_start_loc, "b_seq_start_loc"), (seq_len_tensor, "seq_len_tensor"),
        (lora_indices_tensor, "lora_indices_tensor")])
    for t, n in ((inputs, "inputs"), (lora_b_weights, "lora_b_weights")):
        if t.device != device:
            raise ValueError(f"{n} must be on {device}")
    if start.shape[0] < batches or lens.shape[0] < batches or idx.shape[0] < batches:
        raise ValueError("segment metadata shorter than batches")
    x = _matrix(inputs, "inputs")
    w = _stack(lora_b_weights, "lora_b_weights")
    out = _matrix(output_tensor, "output_tensor")
    stream = _stream(device)
    st = _call_on(device, lib.sgmv_expand_slice, x, w, out, start.data_ptr(), lens.data_ptr(),
                  idx.data_ptr(), int(batches), int(max_seq_length), int(slice_offset),
                  int(slice_size), int(bool(add_inputs)), stream)
    if st != SGMV_OK:
        _raise(st)
    return output_tensor


def sgmv_expand_multi_slice(slices: Sequence[Tuple[object, object, int]], output_tensor,
                            b_seq_start_loc, seq_len_tensor, lora_indices_tensor, batches: int,
                            max_seq_length: int, add_inputs: bool = False):
    """Several slices of one fused output (e.g. Q, K, V) in one launch.

    ``slices``: sequence of (inputs, lora_b_weights, slice_offset); each
    slice's size is its lora_b_weights.size(-2).  Bit-identical to one
    sgmv_expand_slice call per slice."""
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1..{MAX_SLICES} slices, got {len(slices)}")
    device, (start, lens, idx) = _common(output_tensor, [
        (b_seq_start_loc, "b_seq_start_loc"), (seq_len_tensor, "seq_len_tensor"),
        (lora_indices_tensor, "lora_indices_tensor")])
    if start.shape[0] < batches or lens.shape[0] < batches or idx.shape[0] < batches:
        raise ValueError("segment metadata shorter than batches")
    arr = (SliceDesc * len(slices))()
    for i, (x, w, off) in enumerate(slices):
        if x.device != device or w.device != device:
            raise ValueError(f"slice {i} must be on {device}")
        st = _stack(w, f"slice {i} lora_b")
        arr[i] = SliceDesc(_matrix(x, f"slice {i} inputs"), st, int(off), st.rows)
    out = _matrix(output_tensor, "output_tensor")
    stream = _stream(device)
    rc = _call_on(device, lib.sgmv_expand_multi_slice, arr, len(slices), out, start.data_ptr(),
                  lens.data_ptr(), idx.data_ptr(), int(batches), int(max_seq_length),
                  int(bool(add_inputs)), stream)
    if rc != SGMV_OK:
        _raise(rc)
    return output_tensor


def bgmv_expand_slice(inputs, lora_b_weights, output_tensor, lora_indices_tensor, slice_offset: int,
                      slice_size: int, add_inputs: bool = False):
    """Per-token form: output_tensor[t, slice_offset:slice_offset + slice_size]
    (+)= inputs[t] @ lora_b_weights[lora_indices[t]].T for every token t with
    index != -1.  Enqueued on the current stream."""
    device, (idx,) = _common(output_tensor, [(lora_indices_tensor, "lora_indices_tensor")])
    for t, n in ((inputs, "inputs"), (lora_b_weights, "lora_b_weights")):
        if t.device != device:
            raise ValueError(f"{n} must be on {device}")
    if idx.shape[0] < output_tensor.shape[0]:
        raise ValueError("lora_indices_tensor shorter than the number of tokens")
    x = _matrix(inputs, "inputs")
    w = _stack(lora_b_weights, "lora_b_weights")
    out = _matrix(output_tensor, "output_tensor")
    stream = _stream(device)
    st = _call_on(device, lib.sgmv_bgmv_expand_slice, x, w, out, idx.data_ptr(),
                  int(slice_offset), int(slice_size), int(bool(add_inputs)), stream)
    if st != SGMV_OK:
        _raise(st)
    return output_tensor


def _stack_a(w, what: str) -> Stack:
    if w.dim() != 3:
        raise ValueError(f"{what} must be (lora_num, rank, hidden), got {tuple(w.shape)}")
    if not w.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return Stack(w.data_ptr(), _dtype_code(w), w.shape[0], w.shape[1], w.shape[2])


def shrink_workspace_bytes(device=None) -> int:
    """Bytes of the workspace the shrink calls take on `device` (default:
    the current one)."""
    device = _torch.device("cuda", _torch.cuda.current_device()) if device is None else \
        _torch.device(device)
    n = ctypes.c_size_t()
    rc = _call_on(device, lib.sgmv_shrink_workspace_bytes, ctypes.byref(n))
    if rc != SGMV_OK:
        _raise(rc)
    return n.value


# One zero-filled shrink workspace per device, made on first use.
_WORKSPACES = {}


def _workspace(device, workspace):
    """(pointer, bytes) for a shrink call's `workspace` argument: True = this
    device's shared buffer (made and zero-filled on first use; a first use
    inside a graph capture runs without one, since the fill would run only at
    replay), None or False = none, a uint8 tensor = the caller's buffer (zero
    before its first use)."""
    if workspace is None or workspace is False:
        return None, 0
    if workspace is True:
        ws = _WORKSPACES.get(device.index)
        if ws is None:
            if _torch.cuda.is_current_stream_capturing():
                return None, 0
            ws = _torch.zeros(shrink_workspace_bytes(device), dtype=_torch.uint8, device=device)
            _torch.cuda.synchronize(device)
            _WORKSPACES[device.index] = ws
        return ws.data_ptr(), ws.numel()
    if not _torch.is_tensor(workspace) or workspace.device != device or \
            workspace.dtype != _torch.uint8 or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous uint8 tensor on {device}")
    return workspace.data_ptr(), workspace.numel()


def sgmv_shrink(inputs, lora_a_weights, output_tensor, b_seq_start_loc, seq_len_tensor,
                lora_indices_tensor, batches: int, max_seq_length: int, scaling: float = 1.0,
                workspace=True):
    """LoRA-A projection, in place: output_tensor[start_b + m] =
    scaling * inputs[start_b + m] @ lora_a_weights[lora_indices[b]].T for every
    segment b with index != -1 (other rows untouched); lora_a_weights is
    (lora_num, rank, hidden).  Enqueued on the current stream.  `workspace`:
    True (the device's shared buffer: calls that may run concurrently on
    other streams pass buffers of their own), None (large batches run
    unbalanced) or a zero-initialised uint8 tensor of shrink_workspace_bytes()."""
    return sgmv_shrink_multi_slice(inputs, [(lora_a_weights, output_tensor)], b_seq_start_loc,
                                   seq_len_tensor, lora_indices_tensor, batches, max_seq_length,
                                   scaling, workspace)


def _shrink_args(inputs, slices, b_seq_start_loc, seq_len_tensor, lora_indices_tensor,
                 batches):
    """(device, inputs matrix, slice descriptors, start, lens, idx) of a shrink call."""
    if not 1 <= len(slices) <= MAX_SLICES:
        raise ValueError(f"1..{MAX_SLICES} slices, got {len(slices)}")
    device, (start, lens, idx) = _common(inputs, [
        (b_seq_start_loc, "b_seq_start_loc"), (seq_len_tensor, "seq_len_tensor"),
        (lora_indices_tensor, "lora_indices_tensor")])
    if start.shape[0] < batches or lens.shape[0] < batches or idx.shape[0] < batches:
        raise ValueError("segment metadata shorter than batches")
    arr = (ShrinkSliceDesc * len(slices))()
    for i, (w, o) in enumerate(slices):
        if w.device != device or o.device != device:
            raise ValueError(f"slice {i} must be on {device}")
        arr[i] = ShrinkSliceDesc(_stack_a(w, f"slice {i} lora_a"), _matrix(o, f"slice {i} output"))
    return device, _matrix(inputs, "inputs"), arr, start, lens, idx


def sgmv_shrink_multi_slice(inputs, slices: Sequence[Tuple[object, object]], b_seq_start_loc,
                            seq_len_tensor, lora_indices_tensor, batches: int,
                            max_seq_length: int, scaling: float = 1.0, workspace=True):
    """Several LoRA-A projections of the same inputs (e.g. Q, K, V) reading
    the inputs once.  ``slices``: sequence of (lora_a_weights, output_tensor).
    Bit-identical to one sgmv_shrink call per slice with the same
    `workspace` choice."""
    device, x, arr, start, lens, idx = _shrink_args(inputs, slices, b_seq_start_loc,
                                                    seq_len_tensor, lora_indices_tensor, batches)
    ws, ws_bytes = _workspace(device, workspace)
    stream = _stream(device)
    rc = _call_on(device, lib.sgmv_shrink_multi_slice, x, arr, len(slices), start.data_ptr(),
                  lens.data_ptr(), idx.data_ptr(), int(batches), int(max_seq_length),
                  float(scaling), ws, ws_bytes, stream)
    if rc != SGMV_OK:
        _raise(rc)
    return [o for _, o in slices]


def sgmv_shrink_multi_slice_noalloc(inputs, slices: Sequence[Tuple[object, object]],
                                    b_seq_start_loc, seq_len_tensor, lora_indices_tensor,
                                    batches: int, max_seq_length: int, scaling: float = 1.0):
    """sgmv_shrink_multi_slice on the library's static workspace (for callers
    that cannot allocate; calls that may overlap on one device race on it).
    Equal bit for bit to sgmv_shrink_multi_slice with a workspace."""
    device, x, arr, start, lens, idx = _shrink_args(inputs, slices, b_seq_start_loc,
                                                    seq_len_tensor, lora_indices_tensor, batches)
    stream = _stream(device)
    rc = _call_on(device, lib.sgmv_shrink_multi_slice_noalloc, x, arr, len(slices),
                  start.data_ptr(), lens.data_ptr(), idx.data_ptr(), int(batches),
                  int(max_seq_length), float(scaling), stream)
    if rc != SGMV_OK:
        _raise(rc)
    return [o for _, o in slices]


def sgmv_fused_shrink_expand(inputs, slices: Sequence[Tuple[object, object, int]], output_tensor,
                             b_seq_start_loc, seq_len_tensor, lora_indices_tensor, batches: int,
                             max_seq_length: int, scaling: float = 1.0,
                             add_inputs: bool = False):
    """The LoRA-A projection and the expand of its result in one launch, for
    the slices of a fused layer: for each (lora_a_weights (lora_num, rank,
    hidden), lora_b_weights (lora_num, slice_size, rank), slice_offset),
    output_tensor[start_b + m, off:off + slice_size] (+)= rne_w(scaling *
    inputs[start_b + m] @ lora_a[idx].T) @ lora_b[idx].T, the projection
    rounded to the weights' 16-bit dtype and never stored.  Equal to
    sgmv_shrink_multi_slice into weight-dtype outputs followed by
    sgmv_expand_multi_slice.  Enqueued on the current stream."""
    if not 1 <= len(slices) <= MAX_FUSED_SLICES:
        raise ValueError(f"1..{MAX_FUSED_SLICES} slices, got {len(slices)}")
    device, (start, lens, idx) = _common(output_tensor, [
        (b_seq_start_loc, "b_seq_start_loc"), (seq_len_tensor, "seq_len_tensor"),
        (lora_indices_tensor, "lora_indices_tensor")])
    if inputs.device != device:
        raise ValueError(f"inputs must be on {device}")
    if start.shape[0] < batches or lens.shape[0] < batches or idx.shape[0] < batches:
        raise ValueError("segment metadata shorter than batches")
    arr = (FusedSliceDesc * len(slices))()
    for i, (a, w, off) in enumerate(slices):
        if a.device != device or w.device != device:
            raise ValueError(f"slice {i} must be on {device}")
        arr[i] = FusedSliceDesc(_stack_a(a, f"slice {i} lora_a"), _stack(w, f"slice {i} lora_b"),
                                int(off))
    x = _matrix(inputs, "inputs")
    out = _matrix(output_tensor, "output_tensor")
    stream = _stream(device)
    rc = _call_on(device, lib.sgmv_fused_shrink_expand, x, arr, len(slices), out,
                  start.data_ptr(), lens.data_ptr(), idx.data_ptr(), int(batches),
                  int(max_seq_length), float(scaling), int(bool(add_inputs)), stream)
    if rc != SGMV_OK:
        _raise(rc)
    return output_tensor


def abi_version() -> int:
    return lib.sgmv_abi_version()


__all__ = ["sgmv_expand_slice", "sgmv_expand_multi_slice", "bgmv_expand_slice", "sgmv_shrink",
           "shrink_workspace_bytes", "sgmv_shrink_multi_slice_noalloc",
           "sgmv_shrink_multi_slice", "sgmv_fused_shrink_expand", "abi_version", "SgmvError",
           "lib", "Matrix", "Stack", "SliceDesc", "ShrinkSliceDesc", "FusedSliceDesc",
           "EXPORTED_SYMBOLS", "LIBRARY_PATH"]
