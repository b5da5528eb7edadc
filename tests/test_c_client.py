"""The C ABI used from plain C: tests/c/abi_host.c is compiled with gcc against include/kvq.h,
linked against the built libkvq.so and run (host-only entry points; no GPU needed)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "decode_attention_sub_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_plain_c_client(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libkvq.so")):
        pytest.fail("libkvq.so is not built (python -c 'import __graft_entry__ as g; g.build()')")
    exe = str(tmp_path / "abi_host")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", LIBDIR, "-lkvq",
                    f"-Wl,-rpath,{LIBDIR}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count("ok ") == 12
