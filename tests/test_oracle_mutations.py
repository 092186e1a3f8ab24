"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of oracle/sgmv_oracle.c (on the CPU), builds it, and runs
the oracle's pin tests against that build in a child process; at least one
pin must fail.  (Planting is done here, in test code; the oracle source is
never changed.)"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCE = os.path.join(ROOT, "oracle", "sgmv_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_shrink_pins.py",
        "tests/test_oracle_nonfinite.py", "tests/test_oracle_fused_pins.py",
        "tests/test_oracle_codecs.py"]

MUTATIONS = {
    # the weight operand transposed (row k, column n of a slice)
    "transposed_weight": ("r += xrow[k] * wrow[k];",
                          "r += xrow[k] * wval[a * s->N * K + k * s->N + n];"),
    "dropped_prior": ("double r = add ? prior : 0.0;", "double r = 0.0;"),
    "wrong_adapter": ("const int64_t a = c->idx[b];\n    for (int64_t k = 0; k < c->K; ++k) xrow[k]",
                      "const int64_t a = 0;\n    for (int64_t k = 0; k < c->K; ++k) xrow[k]"),
    "missing_cast": ("if (s->x_dtype == ORC_F32) return orc_decode(s->w_dtype, orc_encode(s->w_dtype, v));",
                     ""),
    "sign_flip": ("r += xrow[k] * wrow[k];", "r -= xrow[k] * wrow[k];"),
    "ties_away": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
                  "if (frac >= 0.5) r += 1.0;"),
    "dropped_rank_term": ("for (int64_t k = 0; k < K; ++k) r += xrow[k] * wrow[k];",
                          "for (int64_t k = 0; k + 1 < K; ++k) r += xrow[k] * wrow[k];"),
    # one row past every segment written as well (where the row exists)
    "extra_row": ("for (int64_t m = 0; m < lens[b]; ++m) {",
                  "for (int64_t m = 0; m < lens[b] + (start[b] + lens[b] < T ? 1 : 0); ++m) {"),
    "shrink_dropped_scale": ("r *= c->scale;", ""),
    "shrink_wrong_row": ("const int64_t row_a = (a * c->K + k) * c->H;",
                         "const int64_t row_a = (a * c->K + (k + 1) % c->K) * c->H;"),
    "nonfinite_any_inf": ("const int ok = is_nan_bits(od, rb) ? is_nan_bits(od, cb) : (cb == rb);",
                          "const int ok = is_nan_bits(od, rb) ? is_nan_bits(od, cb) : is_nonfinite_bits(od, cb);"),
    "overflow_saturates": ("if (eu > bias) return sbit | (emask << mb);",
                           "if (eu > bias) return sbit | ((emask - 1) << mb) | ((1u << mb) - 1);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SOURCE).read()
    assert text.count(old) == 1, f"mutation site of {name} not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import build as oracle_build
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-I", os.path.join(ROOT, "oracle"), str(src),
                    "-o", str(lib), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, ORACLE_LIBRARY=str(lib))
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                          "-p", "no:cacheprovider", *PINS], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 1, (f"{name}: no pin failed (rc {res.returncode})\n"
                                 f"{res.stdout[-2000:]}{res.stderr[-2000:]}")
    assert "failed" in res.stdout
