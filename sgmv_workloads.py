"""Seeded synthetic inputs for SGMV expand-slice.

This module only draws inputs: segment metadata, weights, inputs and the
prior output.  It holds none of the operation's arithmetic and is shared by
the oracle side (tests) and the GPU side (tests, benchmark) so that both see
the same bits.

Storage: 16-bit values are numpy ``uint16`` bit patterns, float32 values are
``float32``.  Normals are drawn in float32 as ``rng.standard_normal * sigma``
and rounded once to the storage type (numpy's float16 cast, torch's bfloat16
cast; both round to nearest even).

The five named workloads follow the shapes the SGMV expand-slice wiki page's
usage describes (fused QKV and gate/up slices, packed variable-length
prefill segments, index -1 for "no LoRA"); their sizes, distributions and
draw order are fixed here:

    seq_lens -> (placement) -> lora_indices -> lora_B per slice
             -> inputs per slice -> prior output
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Sequence

import numpy as np

DTYPE_BYTES = {"f16": 2, "bf16": 2, "f32": 4}


def _to_storage(values_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype (round to nearest even)."""
    values_f32 = np.asarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return np.ascontiguousarray(values_f32)
    if dtype == "f16":
        return np.ascontiguousarray(values_f32.astype(np.float16).view(np.uint16))
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(values_f32)).to(torch.bfloat16)
        return np.ascontiguousarray(t.view(torch.int16).numpy().view(np.uint16))
    raise ValueError(dtype)


def normal(rng: np.random.Generator, shape, sigma: float, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        v = v * np.float32(sigma)
    return _to_storage(v, dtype)


def integers_as(rng: np.random.Generator, shape, lo: int, hi: int, dtype: str) -> np.ndarray:
    """Small integers in [lo, hi] stored exactly in ``dtype``."""
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return _to_storage(v, dtype)


@dataclass
class SliceInput:
    x: np.ndarray          # (T, K) or wider rows (row stride >= K)
    x_dtype: str
    w: np.ndarray          # (L, N, K) contiguous
    w_dtype: str
    offset: int

    @property
    def N(self) -> int:
        return int(self.w.shape[1])


@dataclass
class Workload:
    name: str
    slices: List[SliceInput]
    out0: np.ndarray       # (T, H) prior output
    out_dtype: str
    start: np.ndarray      # int64 [B]  (b_seq_start_loc)
    lens: np.ndarray       # int64 [B]  (seq_len_tensor)
    idx: np.ndarray        # int64 [B]  (lora_indices_tensor)
    add: bool
    K: int
    L: int
    seed: int = 0
    notes: Dict[str, object] = field(default_factory=dict)
    per_token: bool = False   # BGMV form: segment t is row t alone (start t, length 1)

    @property
    def T(self) -> int:
        return int(self.out0.shape[0])

    @property
    def H(self) -> int:
        return int(self.out0.shape[1])

    @property
    def batches(self) -> int:
        return int(len(self.lens))

    @property
    def max_seq_len(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0

    def active_mask(self) -> np.ndarray:
        return (self.idx != -1) & (self.lens > 0)


def exclusive_cumsum(lens: Sequence[int]) -> np.ndarray:
    """Start rows of packed segments: [4, 6] -> [0, 4]."""
    lens = np.asarray(lens, dtype=np.int64)
    out = np.zeros_like(lens)
    if len(lens) > 1:
        out[1:] = np.cumsum(lens)[:-1]
    return out


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

def tiny_ref(seed: int = 0) -> Workload:
    """2 sequences of lengths [4, 6] (starts [0, 4]); rank 8; 2 adapters;
    lora_B (2, 64, 8) fp16 N(0, 0.02); input (10, 8) fp16 N(0, 1); output
    (10, 192) fp16 prefilled N(0, 1); slice [64, 128); indices [1, -1];
    overwrite."""
    rng = np.random.default_rng(seed)
    lens = np.array([4, 6], dtype=np.int64)
    idx = np.array([1, -1], dtype=np.int64)
    K, N, H, L, off = 8, 64, 192, 2, 64
    T = int(lens.sum())
    w = normal(rng, (L, N, K), 0.02, "f16")
    x = normal(rng, (T, K), 1.0, "f16")
    out0 = normal(rng, (T, H), 1.0, "f16")
    return Workload("tiny_ref", [SliceInput(x, "f16", w, "f16", off)], out0, "f16",
                    exclusive_cumsum(lens), lens, idx, False, K, L, seed)


def llama7b_q_proj(seed: int = 0) -> Workload:
    """Single slice, Llama-7B-like q_proj: 8 sequences with lengths uniform in
    [64, 512]; rank 16; hidden 4096 = slice; 4 adapters, lora_B (4, 4096, 16)
    bf16 N(0, 0.02); input bf16 N(0, 1); indices uniform in {-1, 0..3};
    accumulate onto a bf16 N(0, 1) output."""
    rng = np.random.default_rng(seed)
    B, K, N, L = 8, 16, 4096, 4
    lens = rng.integers(64, 513, size=B).astype(np.int64)
    idx = rng.integers(-1, L, size=B).astype(np.int64)
    T = int(lens.sum())
    w = normal(rng, (L, N, K), 0.02, "bf16")
    x = normal(rng, (T, K), 1.0, "bf16")
    out0 = normal(rng, (T, N), 1.0, "bf16")
    return Workload("llama7b_q_proj", [SliceInput(x, "bf16", w, "bf16", 0)], out0, "bf16",
                    exclusive_cumsum(lens), lens, idx, True, K, L, seed)


QKV_SLICES = ((0, 4096), (4096, 1024), (5120, 1024))


def gqa_qkv(seed: int = 0, shared_input: bool = False) -> Workload:
    """Fused GQA QKV: output width 6144 = Q [0, 4096) + K [4096, 5120) +
    V [5120, 6144); rank 32; 16 adapters with per-slice lora_B bf16
    N(0, 0.02); 32 sequences with lengths log-uniform in [1, 2048]; per-slice
    inputs bf16 N(0, 1) (one shared input if ``shared_input``); accumulate
    onto a bf16 N(0, 1) output; every sequence has an adapter."""
    rng = np.random.default_rng(seed)
    B, K, L, H = 32, 32, 16, 6144
    u = rng.uniform(0.0, math.log(2048.0), size=B)
    lens = np.clip(np.rint(np.exp(u)), 1, 2048).astype(np.int64)
    idx = rng.integers(0, L, size=B).astype(np.int64)
    T = int(lens.sum())
    ws = [normal(rng, (L, n, K), 0.02, "bf16") for _, n in QKV_SLICES]
    if shared_input:
        x = normal(rng, (T, K), 1.0, "bf16")
        xs = [x, x, x]
    else:
        xs = [normal(rng, (T, K), 1.0, "bf16") for _ in QKV_SLICES]
    out0 = normal(rng, (T, H), 1.0, "bf16")
    slices = [SliceInput(xs[i], "bf16", ws[i], "bf16", QKV_SLICES[i][0]) for i in range(3)]
    return Workload("gqa_qkv", slices, out0, "bf16", exclusive_cumsum(lens), lens, idx, True,
                    K, L, seed, {"shared_input": shared_input})


def mlp_gate_up(seed: int = 0) -> Workload:
    """MLP gate/up: output width 28672, slice [14336, 28672); rank 64; 64
    adapters, lora_B (64, 14336, 64) bf16 N(0, 0.02); 64 sequences with
    lengths uniform in [1, 512] (about 16384 tokens); input float32 N(0, 1)
    cast to bf16 for the products; bf16 output (prefilled N(0, 1) so the
    untouched half is checked); overwrite; every sequence has an adapter."""
    rng = np.random.default_rng(seed)
    B, K, N, H, L, off = 64, 64, 14336, 28672, 64, 14336
    lens = rng.integers(1, 513, size=B).astype(np.int64)
    idx = rng.integers(0, L, size=B).astype(np.int64)
    T = int(lens.sum())
    w = normal(rng, (L, N, K), 0.02, "bf16")
    x = normal(rng, (T, K), 1.0, "f32")
    out0 = normal(rng, (T, H), 1.0, "bf16")
    return Workload("mlp_gate_up", [SliceInput(x, "f32", w, "bf16", off)], out0, "bf16",
                    exclusive_cumsum(lens), lens, idx, False, K, L, seed)


def skewed_mixed(seed: int = 0) -> Workload:
    """Skewed mixed batch: 256 sequences, one of 8192 tokens and 255 of 1..16
    tokens, in shuffled order; rank 128; slice = hidden = 8192; 128 adapters,
    lora_B fp16 N(0, 0.02); input fp16 N(0, 1); indices uniform over adapters
    with exactly 64 (25%) of the short sequences set to -1; accumulate onto
    an fp16 N(0, 1) output."""
    rng = np.random.default_rng(seed)
    B, K, N, L = 256, 128, 8192, 128
    short = rng.integers(1, 17, size=B - 1)
    unordered = np.concatenate([[8192], short]).astype(np.int64)
    perm = rng.permutation(B)
    lens = unordered[perm]
    idx = rng.integers(0, L, size=B).astype(np.int64)
    short_positions = np.nonzero(perm != 0)[0]
    off_positions = rng.choice(short_positions, size=64, replace=False)
    idx[off_positions] = -1
    T = int(lens.sum())
    w = normal(rng, (L, N, K), 0.02, "f16")
    x = normal(rng, (T, K), 1.0, "f16")
    out0 = normal(rng, (T, N), 1.0, "f16")
    return Workload("skewed_mixed", [SliceInput(x, "f16", w, "f16", 0)], out0, "f16",
                    exclusive_cumsum(lens), lens, idx, True, K, L, seed)


def bgmv_decode(seed: int = 0) -> Workload:
    """Per-token (BGMV) decode step with q_proj shapes: 256 tokens, one per
    sequence; rank 16; hidden 4096 = slice; 32 adapters, lora_B (32, 4096, 16)
    bf16 N(0, 0.02); input bf16 N(0, 1); indices uniform in {-1, 0..31};
    accumulate onto a bf16 N(0, 1) output."""
    rng = np.random.default_rng(seed)
    T, K, N, L = 256, 16, 4096, 32
    idx = rng.integers(-1, L, size=T).astype(np.int64)
    w = normal(rng, (L, N, K), 0.02, "bf16")
    x = normal(rng, (T, K), 1.0, "bf16")
    out0 = normal(rng, (T, N), 1.0, "bf16")
    return Workload("bgmv_decode", [SliceInput(x, "bf16", w, "bf16", 0)], out0, "bf16",
                    np.arange(T, dtype=np.int64), np.ones(T, dtype=np.int64), idx, True, K, L,
                    seed, per_token=True)


def per_token(idx: Sequence[int], **kw) -> Workload:
    """A per-token (BGMV) workload: token t alone is segment t, with adapter
    idx[t]; other arguments as for custom()."""
    T = len(idx)
    wl = custom([1] * T, idx, start=list(range(T)), T=T, **kw)
    wl.per_token = True
    return wl


def nonfinite(x_dtype: str = "f16", w_dtype: str = "f16", out_dtype: str = "f16",
              add: bool = True, off: int = 8, seed: int = 0) -> Workload:
    """Integer-valued data (x, W in [-3, 3], prior in [-8, 8]) with NaN, +-Inf
    and overflowing values planted in rows of active segments, in weights
    those rows use and in their prior output; also NaN in a row and a prior
    element of the index -1 segment.  Segments: rows 0-5 adapter 0, 6-10
    adapter 1, 11-14 index -1, 15-21 adapter 0; rank 16, slice of 64 columns
    at ``off`` in rows of 80.

    Planted (slice-relative columns):
      x[1][3] = NaN; x[2][0] = +Inf; x[3][0] = +Inf and x[3][1] = -Inf;
      x[16][:] = 6144 (sums of up to 16 * 3 * 6144 = 294912 overflow f16);
      x[17][0] = 3.4e38 when x is float32 (its cast to f16 or bf16 is +Inf);
      W[1][5][2] = NaN; W[1][9][4] = +Inf;
      prior[4][5] = -Inf; prior[5][7] = NaN (overwritten unless add);
      x[12][0] = NaN and prior[13][1] = NaN in the index -1 segment."""
    lens, idx = [6, 5, 4, 7], [0, 1, -1, 0]
    wl = custom(lens, idx, K=16, N=64, H=80, off=off, L=2, x_dtype=x_dtype, w_dtype=w_dtype,
                out_dtype=out_dtype, add=add, seed=seed, values="int", name="nonfinite")
    s = wl.slices[0]
    x, w, o = s.x.copy(), s.w.copy(), wl.out0.copy()

    def put(a, index, value, dtype):
        a[index] = _to_storage(np.array([value], dtype=np.float32), dtype)[0]

    for (r, k), v in {(1, 3): np.nan, (2, 0): np.inf, (3, 0): np.inf, (3, 1): -np.inf,
                      (12, 0): np.nan}.items():
        put(x, (r, k), v, x_dtype)
    for k in range(16):
        put(x, (16, k), 6144.0, x_dtype)
    if x_dtype == "f32":
        x[17, 0] = np.float32(3.4e38)
    put(w, (1, 5, 2), np.nan, w_dtype)
    put(w, (1, 9, 4), np.inf, w_dtype)
    put(o, (4, off + 5), -np.inf, out_dtype)
    put(o, (5, off + 7), np.nan, out_dtype)
    put(o, (13, off + 1), np.nan, out_dtype)
    return Workload("nonfinite", [SliceInput(x, x_dtype, w, w_dtype, off)], o, out_dtype,
                    wl.start, wl.lens, wl.idx, add, wl.K, wl.L, seed)


WORKLOADS: Dict[str, Callable[..., Workload]] = {
    "tiny_ref": tiny_ref,
    "llama7b_q_proj": llama7b_q_proj,
    "gqa_qkv": gqa_qkv,
    "mlp_gate_up": mlp_gate_up,
    "skewed_mixed": skewed_mixed,
    "bgmv_decode": bgmv_decode,
}


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    """Storage array (uint16 bits or float32) -> torch tensor of ``dtype`` on
    ``device`` holding the same bits.  A 2-D column-slice view of a wider
    array becomes the same view of the whole array (row stride kept)."""
    import torch
    if a.ndim == 2 and not a.flags.c_contiguous and a.strides[1] == a.itemsize:
        rs = a.strides[0] // a.itemsize
        full = np.lib.stride_tricks.as_strided(a, shape=(a.shape[0], rs),
                                               strides=(a.strides[0], a.itemsize))
        return to_torch(np.ascontiguousarray(full), dtype, device)[:, :a.shape[1]]
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a).to(device)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return torch.from_numpy(a.view(np.int16)).to(device).view(tdt)


# ---------------------------------------------------------------------------
# Free-form workloads for edge-case tests.
# ---------------------------------------------------------------------------

def custom(lens: Sequence[int], idx: Sequence[int], *, K: int, N: int, H: int, off: int,
           L: int, x_dtype: str = "bf16", w_dtype: str = "bf16", out_dtype: str = "bf16",
           add: bool = False, seed: int = 0, start: Optional[Sequence[int]] = None,
           T: Optional[int] = None, values: str = "normal", x_pad: int = 0,
           out_pad: int = 0, extra_slices: Sequence[tuple] = (), name: str = "custom") -> Workload:
    """A workload with explicit segments.

    ``values`` is "normal" (x, prior ~ N(0, 1), W ~ N(0, 0.02)) or "int"
    (x, W in [-3, 3], prior in [-8, 8]: every product and partial sum is an
    exactly representable small integer).  ``x_pad`` / ``out_pad`` widen the
    rows (the extra columns are filled too, so strided views can be tested).
    ``extra_slices`` adds (offset, N) slices after the first.
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    start = exclusive_cumsum(lens) if start is None else np.asarray(start, dtype=np.int64)
    if T is None:
        T = int((start + lens).max()) if len(lens) else 0

    def draw(shape, sigma, lo, hi, dtype):
        if values == "int":
            return integers_as(rng, shape, lo, hi, dtype)
        return normal(rng, shape, sigma, dtype)

    slices = []
    for (o, n) in [(off, N), *extra_slices]:
        w = draw((L, n, K), 0.02, -3, 3, w_dtype)
        xfull = draw((T, K + x_pad), 1.0, -3, 3, x_dtype)
        slices.append(SliceInput(xfull[:, :K] if x_pad else xfull, x_dtype, w, w_dtype, o))
    ofull = draw((T, H + out_pad), 1.0, -8, 8, out_dtype)
    out0 = ofull[:, :H] if out_pad else ofull
    return Workload(name, slices, out0, out_dtype, start, lens, idx, add, K, L, seed)


# ---------------------------------------------------------------------------
# LoRA-A projection (shrink) workloads: the step that produces the expand's
# ``inputs`` (total_tokens, rank).  Same segment draws as the expand
# workload they feed; lora_A is (L, K, H_in); one (T, K) output per slice,
# prefilled so that rows the call must leave alone are checked.
# ---------------------------------------------------------------------------

@dataclass
class ShrinkWorkload:
    name: str
    x: np.ndarray          # (T, H_in) or wider rows
    x_dtype: str
    lora_a: List[np.ndarray]   # per slice (L, K, H_in) contiguous
    a_dtype: str
    outs0: List[np.ndarray]    # per slice (T, K) prior output
    out_dtype: str
    start: np.ndarray
    lens: np.ndarray
    idx: np.ndarray
    scale: float
    K: int
    L: int
    seed: int = 0
    notes: Dict[str, object] = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.x.shape[0])

    @property
    def H(self) -> int:
        return int(self.x.shape[1])

    @property
    def batches(self) -> int:
        return int(len(self.lens))

    @property
    def max_seq_len(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0

    def active_mask(self) -> np.ndarray:
        return (self.idx != -1) & (self.lens > 0)


def _shrink_parts(rng, T, H, K, L, n_slices, x_dtype, a_dtype, out_dtype, values="normal",
                  x_pad=0, out_pad=0):
    def draw(shape, sigma, lo, hi, dtype):
        if values == "int":
            return integers_as(rng, shape, lo, hi, dtype)
        return normal(rng, shape, sigma, dtype)

    # lora_A ~ N(0, 1/H) keeps the projection ~ N(0, 1) for x ~ N(0, 1).
    sigma_a = 1.0 / math.sqrt(max(H, 1))
    lora_a = [draw((L, K, H), sigma_a, -3, 3, a_dtype) for _ in range(n_slices)]
    xfull = draw((T, H + x_pad), 1.0, -3, 3, x_dtype)
    x = xfull[:, :H] if x_pad else xfull
    outs0 = []
    for _ in range(n_slices):
        o = draw((T, K + out_pad), 1.0, -8, 8, out_dtype)
        outs0.append(o[:, :K] if out_pad else o)
    return x, lora_a, outs0


def shrink_q_proj(seed: int = 0) -> ShrinkWorkload:
    """LoRA-A projection feeding llama7b_q_proj: its 8 segments and indices;
    hidden 4096 -> rank 16; 4 adapters, bf16 in, weights and out; scale 2
    (alpha 32 over rank 16)."""
    base = llama7b_q_proj(seed)
    rng = np.random.default_rng(seed + 1000)
    H, K, L = 4096, 16, 4
    x, lora_a, outs0 = _shrink_parts(rng, base.T, H, K, L, 1, "bf16", "bf16", "bf16")
    return ShrinkWorkload("shrink_q_proj", x, "bf16", lora_a, "bf16", outs0, "bf16",
                          base.start, base.lens, base.idx, 2.0, K, L, seed)


def shrink_qkv(seed: int = 0) -> ShrinkWorkload:
    """Fused QKV LoRA-A projection feeding gqa_qkv: its 32 segments; hidden
    4096 -> 3 slices of rank 32 from one shared input; 16 adapters; bf16."""
    base = gqa_qkv(seed)
    rng = np.random.default_rng(seed + 1000)
    H, K, L = 4096, 32, 16
    x, lora_a, outs0 = _shrink_parts(rng, base.T, H, K, L, 3, "bf16", "bf16", "bf16")
    return ShrinkWorkload("shrink_qkv", x, "bf16", lora_a, "bf16", outs0, "bf16",
                          base.start, base.lens, base.idx, 1.0, K, L, seed)


def shrink_gate_up(seed: int = 0) -> ShrinkWorkload:
    """Gate/up LoRA-A projection feeding mlp_gate_up: its 64 segments (about
    16k tokens); hidden 4096 -> 2 slices of rank 64; 64 adapters; bf16 input
    and weights, float32 output (the expand's float32 inputs)."""
    base = mlp_gate_up(seed)
    rng = np.random.default_rng(seed + 1000)
    H, K, L = 4096, 64, 64
    x, lora_a, outs0 = _shrink_parts(rng, base.T, H, K, L, 2, "bf16", "bf16", "f32")
    return ShrinkWorkload("shrink_gate_up", x, "bf16", lora_a, "bf16", outs0, "f32",
                          base.start, base.lens, base.idx, 1.0, K, L, seed)


def shrink_skewed(seed: int = 0) -> ShrinkWorkload:
    """LoRA-A projection feeding skewed_mixed: its 256 segments (one of 8192
    tokens, 255 short, 64 without adapter); hidden 8192 -> rank 128; 128
    adapters; fp16."""
    base = skewed_mixed(seed)
    rng = np.random.default_rng(seed + 1000)
    H, K, L = 8192, 128, 128
    x, lora_a, outs0 = _shrink_parts(rng, base.T, H, K, L, 1, "f16", "f16", "f16")
    return ShrinkWorkload("shrink_skewed", x, "f16", lora_a, "f16", outs0, "f16",
                          base.start, base.lens, base.idx, 1.0, K, L, seed)


def shrink_tiny(seed: int = 0) -> ShrinkWorkload:
    """The page's worked example segments (lengths [4, 6] at starts [0, 4],
    indices [1, -1]) through a LoRA-A projection: hidden 64 -> rank 8, 2
    adapters, fp16."""
    rng = np.random.default_rng(seed)
    lens = np.array([4, 6], dtype=np.int64)
    idx = np.array([1, -1], dtype=np.int64)
    x, lora_a, outs0 = _shrink_parts(rng, 10, 64, 8, 2, 1, "f16", "f16", "f16")
    return ShrinkWorkload("shrink_tiny", x, "f16", lora_a, "f16", outs0, "f16",
                          exclusive_cumsum(lens), lens, idx, 1.0, 8, 2, seed)


def shrink_custom(lens: Sequence[int], idx: Sequence[int], *, H: int, K: int, L: int,
                  slices: int = 1, x_dtype: str = "bf16", a_dtype: str = "bf16",
                  out_dtype: str = "bf16", scale: float = 1.0, seed: int = 0,
                  start: Optional[Sequence[int]] = None, T: Optional[int] = None,
                  values: str = "normal", x_pad: int = 0, out_pad: int = 0,
                  name: str = "shrink_custom") -> ShrinkWorkload:
    """A shrink workload with explicit segments (see custom() for ``values``,
    ``x_pad`` and ``out_pad``)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    start = exclusive_cumsum(lens) if start is None else np.asarray(start, dtype=np.int64)
    if T is None:
        T = int((start + lens).max()) if len(lens) else 0
    x, lora_a, outs0 = _shrink_parts(rng, T, H, K, L, slices, x_dtype, a_dtype, out_dtype,
                                     values, x_pad, out_pad)
    return ShrinkWorkload(name, x, x_dtype, lora_a, a_dtype, outs0, out_dtype, start, lens, idx,
                          float(scale), K, L, seed)


SHRINK_WORKLOADS: Dict[str, Callable[..., ShrinkWorkload]] = {
    "shrink_tiny": shrink_tiny,
    "shrink_q_proj": shrink_q_proj,
    "shrink_qkv": shrink_qkv,
    "shrink_gate_up": shrink_gate_up,
    "shrink_skewed": shrink_skewed,
}


# ---------------------------------------------------------------------------
# Fused LoRA delta workloads: the LoRA-A projection of the hidden states and
# the expand of its result into the slices of a fused layer, in one call.
# Same segment draws as the expand workload of the same layer; lora_A ~
# N(0, 1/H) (the projection ~ N(0, 1)), lora_B ~ N(0, 0.02), inputs and
# prior output ~ N(0, 1).
# ---------------------------------------------------------------------------

@dataclass
class FusedWorkload:
    name: str
    x: np.ndarray              # (T, H) hidden states, or wider rows
    x_dtype: str
    lora_a: List[np.ndarray]   # per slice (L, K, H) contiguous
    lora_b: List[np.ndarray]   # per slice (L, N_s, K) contiguous
    w_dtype: str               # dtype of lora_A and lora_B (and of the projection)
    offsets: List[int]         # per slice: first output column
    out0: np.ndarray           # (T, H_out) prior output
    out_dtype: str
    start: np.ndarray
    lens: np.ndarray
    idx: np.ndarray
    scale: float
    add: bool
    K: int
    L: int
    seed: int = 0

    @property
    def T(self) -> int:
        return int(self.x.shape[0])

    @property
    def H(self) -> int:
        return int(self.x.shape[1])

    @property
    def batches(self) -> int:
        return int(len(self.lens))

    @property
    def max_seq_len(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0

    def active_mask(self) -> np.ndarray:
        return (self.idx != -1) & (self.lens > 0)


def _fused_parts(rng, T, H, K, L, slices, H_out, x_dtype, w_dtype, out_dtype, values="normal",
                 x_pad=0, out_pad=0):
    def draw(shape, sigma, lo, hi, dtype):
        if values == "int":
            return integers_as(rng, shape, lo, hi, dtype)
        return normal(rng, shape, sigma, dtype)

    sigma_a = 1.0 / math.sqrt(max(H, 1))
    lora_a = [draw((L, K, H), sigma_a, -2, 2, w_dtype) for _ in slices]
    lora_b = [draw((L, n, K), 0.02, -2, 2, w_dtype) for _, n in slices]
    xfull = draw((T, H + x_pad), 1.0, -2, 2, x_dtype)
    ofull = draw((T, H_out + out_pad), 1.0, -8, 8, out_dtype)
    return (xfull[:, :H] if x_pad else xfull, lora_a, lora_b,
            ofull[:, :H_out] if out_pad else ofull)


def fused_qkv(seed: int = 0) -> FusedWorkload:
    """Fused QKV LoRA delta: the 32 segments of gqa_qkv (lengths
    log-uniform in [1, 2048]); hidden 4096 -> rank 32 -> Q [0, 4096),
    K [4096, 5120), V [5120, 6144); 16 adapters, indices uniform in 0..15;
    bf16 throughout; accumulate onto the prior output."""
    base = gqa_qkv(seed)
    rng = np.random.default_rng(seed + 2000)
    H, K, L = 4096, 32, 16
    x, la, lb, out0 = _fused_parts(rng, base.T, H, K, L, QKV_SLICES, 6144, "bf16", "bf16", "bf16")
    return FusedWorkload("fused_qkv", x, "bf16", la, lb, "bf16", [o for o, _ in QKV_SLICES], out0,
                         "bf16", base.start, base.lens, base.idx, 1.0, True, K, L, seed)


def fused_gate_up(seed: int = 0) -> FusedWorkload:
    """Fused gate/up LoRA delta: the 64 segments of mlp_gate_up (about 16k
    tokens, lengths uniform in [1, 512]); hidden 4096 -> rank 64 -> gate
    [0, 14336) and up [14336, 28672); 64 adapters; bf16 throughout;
    overwrite."""
    base = mlp_gate_up(seed)
    rng = np.random.default_rng(seed + 2000)
    H, K, L = 4096, 64, 64
    sl = ((0, 14336), (14336, 14336))
    x, la, lb, out0 = _fused_parts(rng, base.T, H, K, L, sl, 28672, "bf16", "bf16", "bf16")
    return FusedWorkload("fused_gate_up", x, "bf16", la, lb, "bf16", [o for o, _ in sl], out0,
                         "bf16", base.start, base.lens, base.idx, 1.0, False, K, L, seed)


def fused_q_proj(seed: int = 0) -> FusedWorkload:
    """Fused q_proj LoRA delta on a short prefill batch: the 8 segments of
    llama7b_q_proj (lengths uniform in [64, 512], indices uniform in
    {-1, 0..3}); hidden 4096 -> rank 16 -> one 4096-wide slice; 4 adapters;
    bf16 throughout; accumulate onto the prior output."""
    base = llama7b_q_proj(seed)
    rng = np.random.default_rng(seed + 2000)
    H, K, L = 4096, 16, 4
    sl = ((0, 4096),)
    x, la, lb, out0 = _fused_parts(rng, base.T, H, K, L, sl, 4096, "bf16", "bf16", "bf16")
    return FusedWorkload("fused_q_proj", x, "bf16", la, lb, "bf16", [o for o, _ in sl], out0,
                         "bf16", base.start, base.lens, base.idx, 1.0, True, K, L, seed)


def fused_decode_qkv(seed: int = 0) -> FusedWorkload:
    """Fused QKV LoRA delta on a decode step: 256 one-token segments (the
    per-token layout of bgmv_decode), indices uniform in {-1, 0..31};
    hidden 4096 -> rank 16 -> Q [0, 4096), K [4096, 5120), V [5120, 6144);
    32 adapters; bf16 throughout; accumulate onto the prior output."""
    rng = np.random.default_rng(seed)
    T, H, K, L = 256, 4096, 16, 32
    idx = rng.integers(-1, L, size=T).astype(np.int64)
    lens = np.ones(T, dtype=np.int64)
    x, la, lb, out0 = _fused_parts(rng, T, H, K, L, QKV_SLICES, 6144, "bf16", "bf16", "bf16")
    return FusedWorkload("fused_decode_qkv", x, "bf16", la, lb, "bf16",
                         [o for o, _ in QKV_SLICES], out0, "bf16", exclusive_cumsum(lens), lens,
                         idx, 1.0, True, K, L, seed)


def fused_custom(lens: Sequence[int], idx: Sequence[int], *, H: int, K: int, L: int,
                 slices: Sequence[tuple], H_out: int, x_dtype: str = "bf16",
                 w_dtype: str = "bf16", out_dtype: str = "bf16", add: bool = False,
                 scale: float = 1.0, seed: int = 0, start: Optional[Sequence[int]] = None,
                 T: Optional[int] = None, values: str = "normal", x_pad: int = 0,
                 out_pad: int = 0, name: str = "fused_custom") -> FusedWorkload:
    """A fused workload with explicit segments and (offset, N) slices;
    ``values`` "int" draws x, lora_A, lora_B in [-2, 2] and the prior in
    [-8, 8]."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    start = exclusive_cumsum(lens) if start is None else np.asarray(start, dtype=np.int64)
    if T is None:
        T = int((start + lens).max()) if len(lens) else 0
    x, la, lb, out0 = _fused_parts(rng, T, H, K, L, slices, H_out, x_dtype, w_dtype, out_dtype,
                                   values, x_pad, out_pad)
    return FusedWorkload(name, x, x_dtype, la, lb, w_dtype, [o for o, _ in slices], out0,
                         out_dtype, start, lens, idx, float(scale), add, K, L, seed)


FUSED_WORKLOADS: Dict[str, Callable[..., FusedWorkload]] = {
    "fused_qkv": fused_qkv,
    "fused_gate_up": fused_gate_up,
    "fused_q_proj": fused_q_proj,
    "fused_decode_qkv": fused_decode_qkv,
}
