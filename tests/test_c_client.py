"""examples/sgmv_c_client's own argument and file checks, which end the
program before any HIP call (no GPU needed)."""
import os

import numpy as np

import sgmv_workloads as W
from c_client_util import client_path, run_client, write_expand


def test_client_is_built_and_links_the_in_tree_library():
    import subprocess
    out = subprocess.run(["ldd", client_path()], capture_output=True, text=True).stdout
    lib = next(l for l in out.splitlines() if "libsgmv.so" in l)
    assert os.path.realpath(lib.split("=>")[1].split("(")[0].strip()) == os.path.realpath(
        os.path.join(os.path.dirname(client_path()), "..", "libsgmv.so"))


def test_usage_errors(tmp_path):
    import subprocess
    r = subprocess.run([client_path()], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    r = run_client("transpose", tmp_path, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr
    for mode in ("multi", "shrink", "fused"):
        (tmp_path / "problem.txt").write_text("1 2\n")
        r = run_client(mode, tmp_path, timeout=60)
        assert r.returncode == 1 and f"bad {mode} problem.txt" in r.stderr


def test_missing_and_malformed_files(tmp_path):
    r = run_client("expand", tmp_path, timeout=60)          # no problem.txt
    assert r.returncode == 1 and "problem.txt" in r.stderr
    (tmp_path / "problem.txt").write_text("1 2 3\n")
    r = run_client("expand", tmp_path, timeout=60)
    assert r.returncode == 1 and "bad expand problem.txt" in r.stderr
    wl = W.tiny_ref(0)
    write_expand(tmp_path, wl)
    x = np.fromfile(tmp_path / "x.bin", dtype=np.uint8)
    x[:-2].tofile(tmp_path / "x.bin")                        # two bytes short
    r = run_client("expand", tmp_path, timeout=60)
    assert r.returncode == 1 and "x.bin does not hold" in r.stderr
