"""The C ABI without a GPU: the library loads, exports exactly what
include/sgmv.h declares, and rejects every host-checkable violation of the
I/O Contract before any HIP call (wiki page "Implementation: Predibase Lorax
SGMV Expand Slice Kernel", I/O Contract).  No compute call is made here."""
import os
import re

import pytest

import segmented_gather_gemm_amd as sg
from segmented_gather_gemm_amd import Matrix, SliceDesc, Stack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgmv.h")

F16, BF16, F32 = 0, 1, 2
OK, INVALID, UNSUPPORTED, HIPERR = 0, 1, 2, 3
FAKE = 0x10000  # never dereferenced: every case below fails (or no-ops) before a launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgmv_[a-z_]+)\s*\(", text)))


def test_exports_match_header():
    names = declared_functions()
    assert names == sorted(sg.EXPORTED_SYMBOLS)
    out = os.popen(f"nm -D --defined-only {sg.LIBRARY_PATH}").read()
    exported = sorted(set(re.findall(r" T (sgmv_[a-z_]+)$", out, flags=re.M)))
    assert exported == names
    for n in names:
        assert hasattr(sg.lib, n)


def test_abi_version_matches_header():
    m = re.search(r"#define SGMV_ABI_VERSION (\d+)", open(HEADER).read())
    assert sg.abi_version() == int(m.group(1))


def call(x=None, w=None, out=None, meta=(FAKE, FAKE, FAKE), batches=2, max_len=6, off=64,
         size=64, add=0):
    x = x or Matrix(FAKE, F16, 10, 8, 8)
    w = w or Stack(FAKE, F16, 2, 64, 8)
    out = out or Matrix(FAKE, F16, 10, 192, 192)
    st = sg.lib.sgmv_expand_slice(x, w, out, *meta, batches, max_len, off, size, add, None)
    return st, sg.lib.sgmv_last_error().decode()


CASES = [
    # (kwargs, status, message fragment)
    (dict(x=Matrix(FAKE, F16, 10, 16, 16)), INVALID, "rank"),
    (dict(size=32), INVALID, "slice_size"),
    (dict(x=Matrix(FAKE, F16, 9, 8, 8)), INVALID, "rows"),
    (dict(off=-1), INVALID, "window"),
    (dict(off=129), INVALID, "window"),
    (dict(out=Matrix(FAKE, F16, 10, 192, 191)), INVALID, "row stride"),
    (dict(x=Matrix(FAKE, F16, 10, 8, 7)), INVALID, "row stride"),
    (dict(x=Matrix(FAKE, F16, 10, 0, 0), w=Stack(FAKE, F16, 2, 64, 0)), INVALID, "inputs shape"),
    (dict(batches=-1), INVALID, "batches"),
    (dict(max_len=-1), INVALID, "max_seq_len"),
    (dict(batches=1 << 20), UNSUPPORTED, "batches"),
    (dict(out=Matrix(FAKE, 7, 10, 192, 192)), INVALID, "dtype"),
    (dict(w=Stack(FAKE, F32, 2, 64, 8)), UNSUPPORTED, "float16 or bfloat16"),
    (dict(x=Matrix(FAKE, BF16, 10, 8, 8)), UNSUPPORTED, "dtype"),
    (dict(x=Matrix(FAKE, F16, 1 << 31, 8, 8), out=Matrix(FAKE, F16, 1 << 31, 192, 192)),
     UNSUPPORTED, "tokens"),
    (dict(x=Matrix(FAKE, F16, 1 << 30, 8, 8), w=Stack(FAKE, F16, 2, 1 << 15, 8),
          out=Matrix(FAKE, F16, 1 << 30, 1 << 15, 1 << 15), off=0, size=1 << 15),
     UNSUPPORTED, "work units"),
    (dict(meta=(0, FAKE, FAKE)), INVALID, "metadata"),
    (dict(out=Matrix(0, F16, 10, 192, 192)), INVALID, "output data"),
    (dict(x=Matrix(0, F16, 10, 8, 8)), INVALID, "null data"),
    (dict(out=Matrix(FAKE, F16, -1, 192, 192)), INVALID, "output shape"),
]


@pytest.mark.parametrize("kw,status,frag", CASES)
def test_invalid_arguments_rejected_before_launch(kw, status, frag):
    st, msg = call(**kw)
    assert st == status, msg
    assert frag in msg


@pytest.mark.parametrize("kw", [dict(batches=0), dict(size=0, w=Stack(FAKE, F16, 2, 0, 8)),
                                dict(x=Matrix(FAKE, F16, 0, 8, 8),
                                     out=Matrix(FAKE, F16, 0, 192, 192)),
                                dict(meta=(0, 0, 0), batches=0)])
def test_no_op_calls_return_ok_without_launch(kw):
    st, msg = call(**kw)
    assert st == OK and msg == ""


def test_error_message_cleared_after_ok():
    assert call(off=-1)[0] == INVALID
    assert call(batches=0) == (OK, "")


def _slice(off, size, rank=8, dt=F16, num=2):
    return SliceDesc(Matrix(FAKE, dt, 10, rank, rank), Stack(FAKE, dt, num, size, rank), off, size)


def multi(slices, n=None, batches=2):
    arr = (SliceDesc * max(len(slices), 1))(*slices)
    st = sg.lib.sgmv_expand_multi_slice(arr, len(slices) if n is None else n,
                                        Matrix(FAKE, F16, 10, 192, 192), FAKE, FAKE, FAKE,
                                        batches, 6, 0, None)
    return st, sg.lib.sgmv_last_error().decode()


def test_multi_slice_checks():
    assert multi([_slice(0, 64), _slice(32, 64)])[0] == INVALID            # overlap
    assert "overlap" in multi([_slice(0, 64), _slice(32, 64)])[1]
    assert multi([_slice(0, 64), _slice(64, 64, rank=16)])[0] == INVALID   # rank differs
    assert multi([_slice(0, 64), _slice(64, 64, num=3)])[0] == INVALID     # lora_num differs
    assert multi([_slice(0, 64), _slice(64, 64, dt=BF16)])[0] == INVALID   # dtype differs
    assert multi([_slice(0, 64)] * 9)[0] == INVALID                         # > 8 slices
    assert multi([_slice(0, 64)], n=0)[0] == INVALID
    assert multi([_slice(0, 64), _slice(160, 64)])[0] == INVALID           # past the output
    assert multi([_slice(0, 64), _slice(64, 64)], batches=0) == (OK, "")
    st = sg.lib.sgmv_expand_multi_slice(None, 1, Matrix(FAKE, F16, 10, 192, 192), FAKE, FAKE,
                                        FAKE, 2, 6, 0, None)
    assert st == INVALID


def bgmv(x=None, w=None, out=None, idx=FAKE, off=64, size=64, add=0):
    x = x or Matrix(FAKE, F16, 10, 8, 8)
    w = w or Stack(FAKE, F16, 2, 64, 8)
    out = out or Matrix(FAKE, F16, 10, 192, 192)
    st = sg.lib.sgmv_bgmv_expand_slice(x, w, out, idx, off, size, add, None)
    return st, sg.lib.sgmv_last_error().decode()


@pytest.mark.parametrize("kw,status,frag", [
    (dict(idx=0), INVALID, "metadata"),
    (dict(x=Matrix(FAKE, F16, 9, 8, 8)), INVALID, "rows"),
    (dict(x=Matrix(FAKE, F16, 10, 16, 16)), INVALID, "rank"),
    (dict(size=32), INVALID, "slice_size"),
    (dict(off=129), INVALID, "window"),
    (dict(w=Stack(FAKE, F32, 2, 64, 8)), UNSUPPORTED, "float16 or bfloat16"),
    (dict(x=Matrix(FAKE, F16, 4001, 8, 8), out=Matrix(FAKE, F16, 4001, 192, 192)),
     UNSUPPORTED, "tokens"),
    (dict(out=Matrix(FAKE, F16, -1, 192, 192)), INVALID, "output shape"),
])
def test_bgmv_invalid_arguments_rejected_before_launch(kw, status, frag):
    st, msg = bgmv(**kw)
    assert st == status, msg
    assert frag in msg


def test_bgmv_no_op_calls():
    assert bgmv(x=Matrix(FAKE, F16, 0, 8, 8), out=Matrix(FAKE, F16, 0, 192, 192)) == (OK, "")
    assert bgmv(size=0, w=Stack(FAKE, F16, 2, 0, 8)) == (OK, "")


def test_python_wrapper_rejects_host_tensors():
    import torch
    x = torch.zeros(10, 8, dtype=torch.float16)
    w = torch.zeros(2, 64, 8, dtype=torch.float16)
    o = torch.zeros(10, 192, dtype=torch.float16)
    m = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU"):
        sg.sgmv_expand_slice(x, w, o, m, m, m, 2, 6, 64, 64)


def test_one_hip_runtime_in_process():
    """libsgmv resolves to the HIP runtime PyTorch already mapped."""
    assert len(sg._hip_runtimes_mapped()) == 1


# --------------------------------------------------------------------------
# LoRA-A projection (shrink).
# --------------------------------------------------------------------------

def shrink(x=None, a=None, out=None, meta=(FAKE, FAKE, FAKE), batches=2, max_len=6, scale=1.0,
           ws=None, ws_bytes=0):
    x = x or Matrix(FAKE, F16, 10, 64, 64)
    a = a or Stack(FAKE, F16, 2, 8, 64)
    out = out or Matrix(FAKE, F16, 10, 8, 8)
    st = sg.lib.sgmv_shrink(x, a, out, *meta, batches, max_len, scale, ws, ws_bytes, None)
    return st, sg.lib.sgmv_last_error().decode()


@pytest.mark.parametrize("kw,status,frag", [
    (dict(a=Stack(FAKE, F16, 2, 8, 32)), INVALID, "hidden"),
    (dict(out=Matrix(FAKE, F16, 10, 16, 16)), INVALID, "output"),
    (dict(out=Matrix(FAKE, F16, 9, 8, 8)), INVALID, "output"),
    (dict(out=Matrix(FAKE, F16, 10, 8, 7)), INVALID, "output"),
    (dict(x=Matrix(FAKE, F16, 10, 64, 63)), INVALID, "row stride"),
    (dict(x=Matrix(FAKE, F16, 10, 0, 0), a=Stack(FAKE, F16, 2, 8, 0)), INVALID, "inputs shape"),
    (dict(a=Stack(FAKE, F16, 2, 0, 64), out=Matrix(FAKE, F16, 10, 0, 0)), INVALID, "lora_a shape"),
    (dict(batches=-1), INVALID, "batches"),
    (dict(max_len=-1), INVALID, "max_seq_len"),
    (dict(batches=1 << 20), UNSUPPORTED, "batches"),
    (dict(x=Matrix(FAKE, 7, 10, 64, 64)), INVALID, "dtype"),
    (dict(a=Stack(FAKE, F32, 2, 8, 64)), UNSUPPORTED, "float16 or bfloat16"),
    (dict(x=Matrix(FAKE, BF16, 10, 64, 64)), UNSUPPORTED, "dtype"),
    (dict(a=Stack(FAKE, F16, 2, 264, 64), out=Matrix(FAKE, F16, 10, 264, 264)), UNSUPPORTED,
     "rank"),
    (dict(x=Matrix(FAKE, F16, 1 << 31, 64, 64), out=Matrix(FAKE, F16, 1 << 31, 8, 8)),
     UNSUPPORTED, "tokens"),
    (dict(meta=(FAKE, 0, FAKE)), INVALID, "metadata"),
    (dict(x=Matrix(0, F16, 10, 64, 64)), INVALID, "inputs data"),
    (dict(out=Matrix(0, F16, 10, 8, 8)), INVALID, "null data"),
])
def test_shrink_invalid_arguments_rejected_before_launch(kw, status, frag):
    st, msg = shrink(**kw)
    assert st == status, msg
    assert frag in msg


def test_shrink_no_op_calls():
    assert shrink(batches=0) == (OK, "")
    assert shrink(x=Matrix(FAKE, F16, 0, 64, 64), out=Matrix(FAKE, F16, 0, 8, 8)) == (OK, "")
    assert shrink(meta=(0, 0, 0), batches=0) == (OK, "")


def test_shrink_multi_slice_checks():
    def sl(rank=8, num=2, dt=F16, odt=F16):
        return sg.ShrinkSliceDesc(Stack(FAKE, dt, num, rank, 64), Matrix(FAKE, odt, 10, rank, rank))

    def multi_shrink(slices, n=None, batches=2):
        arr = (sg.ShrinkSliceDesc * max(len(slices), 1))(*slices)
        st = sg.lib.sgmv_shrink_multi_slice(Matrix(FAKE, F16, 10, 64, 64), arr,
                                            len(slices) if n is None else n, FAKE, FAKE, FAKE,
                                            batches, 6, 1.0, None, 0, None)
        return st, sg.lib.sgmv_last_error().decode()

    assert multi_shrink([sl(), sl(rank=16)])[0] == INVALID
    assert multi_shrink([sl(), sl(num=3)])[0] == INVALID
    assert multi_shrink([sl(), sl(odt=F32)])[0] == INVALID
    assert multi_shrink([sl()] * 9)[0] == INVALID
    assert multi_shrink([sl()], n=0)[0] == INVALID
    assert multi_shrink([sl(), sl()], batches=0) == (OK, "")
    st = sg.lib.sgmv_shrink_multi_slice(Matrix(FAKE, F16, 10, 64, 64), None, 1, FAKE, FAKE, FAKE,
                                        2, 6, 1.0, None, 0, None)
    assert st == INVALID


def test_shrink_noalloc_rejects_a_null_slice_array_first():
    st = sg.lib.sgmv_shrink_multi_slice_noalloc(Matrix(FAKE, F16, 10, 64, 64), None, 1, FAKE,
                                                FAKE, FAKE, 2, 6, 1.0, None)
    assert st == INVALID
    assert "slices pointer" in sg.lib.sgmv_last_error().decode()


def test_shrink_workspace_checks_follow_the_argument_checks():
    """A workspace never masks an argument error, and no-op calls ignore it
    (the workspace's own size and alignment checks need the device's compute
    unit count: tests/test_gpu_shrink.py)."""
    st, msg = shrink(a=Stack(FAKE, F16, 2, 8, 32), ws=FAKE, ws_bytes=1)
    assert st == INVALID and "hidden" in msg
    assert shrink(batches=0, ws=FAKE + 3, ws_bytes=1) == (OK, "")
    assert sg.lib.sgmv_shrink_workspace_bytes(None) == INVALID
    assert "bytes pointer" in sg.lib.sgmv_last_error().decode()


# --------------------------------------------------------------------------
# Fused LoRA delta (shrink and expand in one call).
# --------------------------------------------------------------------------

def fslice(rank=16, hidden=64, n=64, off=0, num=2, dt=F16, bdt=None, a_ptr=FAKE, b_ptr=FAKE):
    return sg.FusedSliceDesc(Stack(a_ptr, dt, num, rank, hidden),
                             Stack(b_ptr, dt if bdt is None else bdt, num, n, rank), off)


def fused(slices=None, x=None, out=None, meta=(FAKE, FAKE, FAKE), batches=2, max_len=6, n=None,
          add=0):
    slices = slices if slices is not None else [fslice()]
    x = x or Matrix(FAKE, F16, 10, 64, 64)
    out = out or Matrix(FAKE, F16, 10, 192, 192)
    arr = (sg.FusedSliceDesc * max(len(slices), 1))(*slices)
    st = sg.lib.sgmv_fused_shrink_expand(x, arr, len(slices) if n is None else n, out, *meta,
                                         batches, max_len, 1.0, add, None)
    return st, sg.lib.sgmv_last_error().decode()


@pytest.mark.parametrize("kw,status,frag", [
    (dict(n=0), INVALID, "num_slices"),
    (dict(slices=[fslice(off=64 * i) for i in range(4)]), INVALID, "num_slices"),
    (dict(slices=[fslice(hidden=32)]), INVALID, "lora_a"),
    (dict(slices=[sg.FusedSliceDesc(Stack(FAKE, F16, 2, 16, 64), Stack(FAKE, F16, 2, 64, 8), 0)]),
     INVALID, "lora_b"),
    (dict(slices=[sg.FusedSliceDesc(Stack(FAKE, F16, 2, 16, 64), Stack(FAKE, F16, 3, 64, 16), 0)]),
     INVALID, "lora_b"),
    (dict(slices=[fslice(off=129)]), INVALID, "window"),
    (dict(slices=[fslice(off=-1)]), INVALID, "window"),
    (dict(slices=[fslice(), fslice(off=32)]), INVALID, "overlap"),
    (dict(slices=[fslice(), fslice(off=64, rank=8)]), INVALID, "match slice 0"),
    (dict(slices=[fslice(), fslice(off=64, num=3)]), INVALID, "match slice 0"),
    (dict(out=Matrix(FAKE, F16, 9, 192, 192)), INVALID, "rows"),
    (dict(out=Matrix(FAKE, F16, 10, 192, 191)), INVALID, "row stride"),
    (dict(x=Matrix(FAKE, F16, 10, 64, 63)), INVALID, "row stride"),
    (dict(batches=-1), INVALID, "batches"),
    (dict(max_len=-1), INVALID, "max_seq_len"),
    (dict(batches=1 << 20), UNSUPPORTED, "batches"),
    (dict(x=Matrix(FAKE, 7, 10, 64, 64)), INVALID, "dtype"),
    (dict(slices=[fslice(dt=F32)]), UNSUPPORTED, "16-bit"),
    (dict(slices=[fslice(bdt=BF16)]), UNSUPPORTED, "16-bit"),
    (dict(x=Matrix(FAKE, BF16, 10, 64, 64)), UNSUPPORTED, "dtype or float32"),
    (dict(meta=(FAKE, 0, FAKE)), INVALID, "metadata"),
    (dict(x=Matrix(0, F16, 10, 64, 64)), INVALID, "null data"),
    (dict(slices=[fslice(a_ptr=0)]), INVALID, "null data"),
    # shapes the fused kernels do not take
    (dict(slices=[fslice(rank=12)]), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(rank=136)]), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(rank=128), fslice(rank=128, off=64), fslice(rank=128, off=128)]),
     UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(n=60)]), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(off=4)]), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(hidden=60)], x=Matrix(FAKE, F16, 10, 60, 60)), UNSUPPORTED,
     "run sgmv_shrink_multi_slice"),
    (dict(x=Matrix(FAKE + 2, F16, 10, 64, 64)), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
    (dict(slices=[fslice(b_ptr=FAKE + 8)]), UNSUPPORTED, "run sgmv_shrink_multi_slice"),
])
def test_fused_invalid_arguments_rejected_before_launch(kw, status, frag):
    st, msg = fused(**kw)
    assert st == status, msg
    assert frag in msg


def test_fused_no_op_calls():
    assert fused(batches=0) == (OK, "")
    assert fused(x=Matrix(FAKE, F16, 0, 64, 64), out=Matrix(FAKE, F16, 0, 192, 192)) == (OK, "")
    assert fused(slices=[fslice(n=0)]) == (OK, "")
    assert fused(meta=(0, 0, 0), batches=0) == (OK, "")
    st = sg.lib.sgmv_fused_shrink_expand(Matrix(FAKE, F16, 10, 64, 64), None, 1,
                                         Matrix(FAKE, F16, 10, 192, 192), FAKE, FAKE, FAKE, 2, 6,
                                         1.0, 0, None)
    assert st == INVALID
