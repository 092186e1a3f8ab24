"""Host-side size predicates of the library's kernel choices and the kernels'
unit assignment (sgmv_limits.h), compiled with the host compiler and checked
at their boundaries (no GPU needed)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "segmented_gather_gemm_amd", "csrc")

PROBE = r"""
#include <stdio.h>
#include <stdlib.h>
#include "sgmv_limits.h"
int main(int argc, char** argv) {
  for (int i = 1; i + 1 < argc; i += 2)
    printf("%d\n", (int)sgmv::limits::shrink_fast_lora_a_fits(atoll(argv[i]), atoll(argv[i + 1])));
  return 0;
}
"""


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    d = tmp_path_factory.mktemp("limits")
    src = d / "probe.cpp"
    src.write_text(PROBE)
    exe = d / "probe"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)

    def run(pairs):
        args = [str(v) for kh in pairs for v in kh]
        out = subprocess.run([str(exe), *args], check=True, capture_output=True, text=True).stdout
        return [bool(int(v)) for v in out.split()]
    return run


def fits(K, H):
    """The bound written out: 16 * next_pow2(ceil(K / 16)) rows of H 16-bit
    elements span less than 2^31 bytes."""
    k16 = 1
    while k16 < -(-K // 16):
        k16 *= 2
    return 16 * k16 * H * 2 < 2 ** 31


@pytest.mark.parametrize("K", [1, 8, 16, 17, 32, 33, 48, 64, 96, 128, 129, 200, 256])
def test_shrink_lora_a_offset_bound(probe, K):
    rows = 16
    while rows < 16 * -(-K // 16):
        rows *= 2
    h_max = (2 ** 31 - 1) // (rows * 2)          # largest hidden size that fits
    cases = [(K, 1), (K, 4096), (K, h_max), (K, h_max + 1), (K, 2 ** 30)]
    got = probe(cases)
    assert got == [fits(k, h) for k, h in cases]
    assert got[2] and not got[3]


def test_shrink_lora_a_offset_bound_named_shapes(probe):
    # rank 256 with hidden 8 Mi (4 GiB per adapter block) and rank 128 with
    # hidden 8 Mi take the generic kernel; the benchmark's shapes stay fast
    cases = [(256, 8 << 20), (128, 8 << 20), (256, (1 << 22) - 1), (256, 1 << 22),
             (16, 4096), (32, 4096), (64, 4096), (128, 8192)]
    assert probe(cases) == [False, False, True, False, True, True, True, True]


SPAN_PROBE = r"""
#include <stdio.h>
#include <stdlib.h>
#include "sgmv_limits.h"
// argv: U G cus -> one line "begin end" per workgroup
int main(int argc, char** argv) {
  const unsigned U = atoi(argv[1]), G = atoi(argv[2]), cus = atoi(argv[3]);
  for (unsigned bid = 0; bid < G; ++bid) {
    const sgmv::limits::UnitSpan s = sgmv::limits::unit_span(U, G, cus, bid);
    printf("%u %u\n", s.begin, s.end);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def spans(tmp_path_factory):
    d = tmp_path_factory.mktemp("spans")
    src = d / "span.cpp"
    src.write_text(SPAN_PROBE)
    exe = d / "span"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)

    def run(U, G, cus):
        out = subprocess.run([str(exe), str(U), str(G), str(cus)], check=True,
                             capture_output=True, text=True).stdout.split()
        v = [int(t) for t in out]
        return list(zip(v[0::2], v[1::2]))
    return run


# (units, grid, compute units): the named shrink and fused launches (e.g. 298
# units of 64 rows in a grid of 320 or 256), grids above and below the unit
# count, grids that are not multiples of 8, empty launches
SPAN_CASES = [(U, G, 256) for U in (0, 1, 7, 8, 9, 84, 182, 192, 255, 256, 257, 298, 319, 512,
                                   1000, 12345)
              for G in (1, 3, 8, 16, 24, 112, 192, 256, 320, 416, 768)] + \
             [(100, 128, 64), (64, 128, 64), (65, 128, 64), (300, 304, 304)]


@pytest.mark.parametrize("U,G,cus", SPAN_CASES)
def test_unit_spans_partition_and_balance(spans, U, G, cus):
    sp = spans(U, G, cus)
    assert len(sp) == G
    # every unit exactly once, each workgroup a contiguous range
    covered = sorted(u for b, e in sp for u in range(b, e))
    assert covered == list(range(U))
    sizes = [e - b for b, e in sp]
    xcd_grid = G >= 16 and G % 8 == 0
    if xcd_grid and U <= G and U <= cus:
        # one unit per workgroup at most, equal shares per XCD (workgroup i on
        # XCD i % 8), and only workgroups of the first wave (i < cus) busy
        assert max(sizes, default=0) <= 1
        per_xcd = [sum(sizes[x::8]) for x in range(8)]
        assert max(per_xcd) - min(per_xcd) <= 1
        assert all(s == 0 for s in sizes[cus:])
        # each XCD's units are one contiguous run, XCD x before XCD x + 1
        for x in range(8):
            own = sorted(u for b, e in sp[x::8] for u in range(b, e))
            assert own == list(range(own[0], own[0] + len(own))) if own else True
    else:
        # contiguous ranges in XCD-major order (plain order for other grids),
        # sizes q or q + 1 with the larger ones first
        order = sorted(range(G), key=lambda i: ((i % 8) * (G // 8) + i // 8) if xcd_grid else i)
        pos = 0
        for i in order:
            b, e = sp[i]
            assert b == pos
            pos = e
        q = U // G
        ordered = [sizes[i] for i in order]
        assert all(s in (q, q + 1) for s in ordered)
        assert ordered == sorted(ordered, reverse=True)


PART_PROBE = r"""
#include <stdio.h>
#include <stdlib.h>
#include "sgmv_limits.h"
// argv: U C G h_steps -> "max_parts W E P counter_bytes workspace_bytes",
// then one line "lo hi" per part, then one line "bid unit part" per
// workgroup bid >= W that runs a part
int main(int argc, char** argv) {
  const unsigned U = atoi(argv[1]), C = atoi(argv[2]), G = atoi(argv[3]), h = atoi(argv[4]);
  const sgmv::limits::PartPlan pl = sgmv::limits::part_plan(U, C, G, h);
  printf("%u %u %u %u %lld %lld\n", sgmv::limits::kShrinkMaxParts, pl.W, pl.E, pl.P,
         (long long)sgmv::limits::shrink_workspace_counter_bytes(C),
         (long long)sgmv::limits::shrink_workspace_bytes(C));
  for (unsigned r = 0; r < pl.P; ++r) {
    const sgmv::limits::StepSpan s = sgmv::limits::part_steps(r, pl.P, h);
    printf("S %d %d\n", s.lo, s.hi);
  }
  for (unsigned bid = pl.W; pl.P && bid < G; ++bid) {
    const sgmv::limits::PartItem it = sgmv::limits::part_item(pl, bid);
    if (it.valid) printf("I %u %u %u\n", bid, it.unit, it.part);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def parts(tmp_path_factory):
    d = tmp_path_factory.mktemp("parts")
    src = d / "part.cpp"
    src.write_text(PART_PROBE)
    exe = d / "part"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", str(src), "-o", str(exe)],
                   check=True)

    def run(U, C, G, h):
        out = subprocess.run([str(exe), str(U), str(C), str(G), str(h)], check=True,
                             capture_output=True, text=True).stdout.split("\n")
        kmax, Wh, E, P, cb, wb = (int(t) for t in out[0].split())
        spans = [tuple(int(t) for t in line.split()[1:]) for line in out[1:] if line[:1] == "S"]
        items = [tuple(int(t) for t in line.split()[1:]) for line in out[1:] if line[:1] == "I"]
        return kmax, Wh, E, P, cb, wb, spans, items
    return run


# (units, compute units, grid, hidden steps): small batches (every unit in
# parts up to C / 2 units), around C and 2 C units (the named shrink batches
# have 298 and 319 units of 64 tokens on 256 compute units), grids too small
# for the parts, hidden sizes with fewer 4-step groups than parts
PART_CASES = [(U, 256, G, h) for U in (0, 1, 32, 64, 65, 85, 100, 128, 129, 255, 256, 257, 298,
                                       319, 320, 384, 385, 450, 512, 513)
              for G in (128, 256, 504, 512, 768) for h in (1, 3, 4, 7, 32, 128, 256)] + \
             [(100, 64, 128, 128), (304 + 30, 304, 608, 128), (20, 12, 24, 128)]


@pytest.mark.parametrize("U,C,G,h", PART_CASES)
def test_part_plan_and_step_spans(parts, U, C, G, h):
    kmax, Wh, E, P, cb, wb, spans, items = parts(U, C, G, h)
    n4 = (h + 3) // 4
    ok = C >= 8 and C % 8 == 0 and 0 < U <= 2 * C
    whole = C if U > C else 0
    want_p = min(C // (U - whole), kmax, n4) if ok else 0
    if want_p < 2 or G < whole + C:
        assert (Wh, E, P) == (0, 0, 0) and spans == [] and items == []
    else:
        # C < U <= 2 C: C whole units, the rest in parts; U <= C / 2: all in parts
        assert (Wh, E, P) == (whole, U - whole, want_p)
        assert U > C or 2 * U <= C
        # every part of every overflow unit exactly once, on the C workgroups
        # after the whole units (one per compute unit); in slot order
        # ((unit - W) P + part) XCD x (bid % 8) holds the x-th contiguous
        # eighth of the parts, taken in order of (bid - W) / 8
        assert sorted((u, r) for _, u, r in items) == \
            [(u, r) for u in range(Wh, Wh + E) for r in range(P)]
        assert all(Wh <= b < Wh + C for b, _, _ in items)
        I = E * P
        share, extra = I // 8, I % 8
        for b, u, r in items:
            x, j = (b - Wh) % 8, (b - Wh) // 8
            assert (u - Wh) * P + r == x * share + min(x, extra) + j
        # spans: contiguous, non-empty, on multiples of 4 steps, covering
        # every hidden step; they depend on (P, h) only
        assert spans[0][0] == 0
        for (lo, hi), (lo2, _) in zip(spans, spans[1:]):
            assert hi == lo2
        for lo, hi in spans:
            assert lo % 4 == 0 and hi % 4 == 0 and hi > lo
        assert spans[-1][1] == 4 * n4 >= h
    # workspace: one 32-bit counter per compute unit (padded to 256 bytes),
    # then one 64 KiB slot per possible part
    assert cb % 256 == 0 and 4 * C <= cb < 4 * C + 256
    assert wb == cb + C * 64 * 256 * 4


def test_shrink_sum_depth_follows_the_kernel_choice():
    """The GPU tests' shrink tolerance uses the most fp32 roundings a product
    passes through: 32 + ceil(H / 32) + 8 where the MFMA kernels run (rank and
    hidden multiples of 8, 16-byte row strides, lora_A span below 2 GiB), the
    hidden size where the generic kernel runs."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    import sgmv_workloads as W
    from gpu_util import shrink_sum_depth
    assert shrink_sum_depth(W.SHRINK_WORKLOADS["shrink_gate_up"](0)) == 32 + 128 + 8
    assert shrink_sum_depth(W.SHRINK_WORKLOADS["shrink_skewed"](0)) == 32 + 256 + 8
    lens, idx = [10, 20], [0, 1]
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=1000, K=24, L=2, seed=1)) == 32 + 32 + 8
    # generic: hidden not a multiple of 8, rank not a multiple of 8, a padded row
    # stride that is not a multiple of 16 bytes; a float32 output padded by 4
    # columns keeps 16-byte rows
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=1001, K=24, L=2, seed=1)) == 1001
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=256, K=7, L=2, seed=1)) == 256
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=1000, K=24, L=2, x_pad=3, seed=1)) == 1000
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=1000, K=24, L=2, out_dtype="f32",
                                            out_pad=4, seed=1)) == 72
    # tiny hidden sizes: never more than H
    assert shrink_sum_depth(W.shrink_custom(lens, idx, H=8, K=8, L=2, seed=1)) == 8


FORM_PROBE = r"""
#include <stdio.h>
#include "sgmv_shrink_launch.h"
int main() {
  for (int k16 = 1; k16 <= 16; k16 *= 2)
    printf("%d %lld\n", k16, (long long)sgmv::shrink_split_t_min_units(k16));
  return 0;
}
"""


def test_shrink_form_threshold_by_rank(tmp_path):
    """The units of 64 tokens from which the shrink (and the fused call,
    which follows it) takes its 64-token form: 129 for one 16-row k tile per
    slice (ranks up to 16), 64 above -- a function of the rank alone."""
    src = tmp_path / "form.cpp"
    src.write_text(FORM_PROBE)
    exe = tmp_path / "form"
    subprocess.run(["g++", "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{CSRC}", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    got = {int(a): int(b) for a, b in (line.split() for line in out.splitlines())}
    assert got == {1: 129, 2: 64, 4: 64, 8: 64, 16: 64}
