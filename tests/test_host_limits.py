"""Host-side size predicates of the library's kernel choices, compiled with
the host compiler and checked at their boundaries (no GPU needed)."""
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
