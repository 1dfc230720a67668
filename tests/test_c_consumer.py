"""The boundary from plain C: tests/c_consumer.c includes include/bsga.h as
C99 (-pedantic, warnings as errors), links libbsga.so and calls the
host-only entry points (version, status strings, block and keep counts, CSR
capacity, workspace size, argument rejection before any launch, head-wise
budgets).  No GPU work, so it runs on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

bsga = pytest.importorskip("block_sparse_global_bsga_amd.bsga", reason="libbsga.so not built")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c99_caller(tmp_path):
    libdir = os.path.dirname(os.path.abspath(bsga.LIB_PATH))
    exe = str(tmp_path / "c_consumer")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_consumer.c"),
           "-L", libdir, "-lbsga", f"-Wl,-rpath,{libdir}", "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
