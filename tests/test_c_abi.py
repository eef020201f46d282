"""The library used from plain C: tests/c/abi_from_c.c is compiled with the
system C compiler against include/*.h, linked with libpagedattn.so and run
(host-side calls only; no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "paged_kv_cache_386_amd")
LIB = os.path.join(LIBDIR, "libpagedattn.so")


@pytest.mark.skipif(not os.path.exists(LIB), reason="libpagedattn.so not built")
@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_c_caller(tmp_path):
    exe = tmp_path / "abi_from_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-L", LIBDIR,
                    "-lpagedattn", f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
