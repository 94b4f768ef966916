"""include/route.h from plain C: a C99 program (tests/c_abi/check_abi.c)
compiles against the header with warnings as errors, links against
libroute.so and gets the documented status codes from every call that
validates before touching the HIP runtime (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

from latent_projection_top_amd import route

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_compiles_as_c_and_links(tmp_path):
    lib_dir = os.path.dirname(route.LIB_PATH)
    exe = tmp_path / "check_abi"
    cc = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi", "check_abi.c"),
          route.LIB_PATH, f"-Wl,-rpath,{lib_dir}", "-o", str(exe)]
    r = subprocess.run(cc, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
