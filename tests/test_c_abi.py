"""The C ABI from a plain C99 program (tests/c_abi/abi_from_c.c): the header
compiles as C with warnings as errors, the library links from C, and the
blob layouts the header documents are the bytes the host packers write.
Host calls only (no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "speculative_verify_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.skipif(not os.path.exists(os.path.join(LIBDIR, "libsvq.so")), reason="libsvq.so not built")
def test_c_client_compiles_links_and_sees_the_documented_layout(tmp_path):
    exe = str(tmp_path / "abi_from_c")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi", "abi_from_c.c"), "-L", LIBDIR, "-lsvq",
           f"-Wl,-rpath,{LIBDIR}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_from_c OK" in r.stdout
