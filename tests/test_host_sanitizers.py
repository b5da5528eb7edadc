"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library's sources are compiled with the sanitizers on the host code only (each
``-fsanitize=`` option goes to the host compilation through ``-Xarch_host``; the gfx950 code
object is built as usual and never runs here), the plain C client tests/c/abi_host.c is built
with the same sanitizers, and the client's host-only calls (byte counts, buffer sizes, workspace
size, argument validation including hostile arguments) must finish without a sanitizer report."""

import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_sub_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_host_abi_under_asan_ubsan(tmp_path):
    from decode_attention_sub_amd import build as B
    objs = []
    procs = []
    for src in B.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        cmd = [HIPCC, *B.FLAGS, *B.PER_FILE.get(src, []), "-O1", "-g", *SAN, "-c",
               os.path.join(CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                      text=True))
        objs.append(obj)
    for pr in procs:
        out, _ = pr.communicate(timeout=600)
        assert pr.returncode == 0, out
    lib = str(tmp_path / "libkvq.so")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-fPIC", "-shared", "-fno-gpu-rdc",
                    "-shared-libsan", *SAN, *objs, "-o", lib], check=True, capture_output=True)
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    assert rt, "no shared AddressSanitizer runtime"
    exe = str(tmp_path / "abi_host_san")
    subprocess.run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-shared-libsan",
                    "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", str(tmp_path), "-lkvq",
                    f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
                    f"-Wl,-rpath,{os.path.dirname(rt[-1])}", "-o", exe],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    log = r.stdout + r.stderr
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
    assert r.returncode == 0, log
    assert "FAIL" not in r.stdout and "hostile arguments rejected" in r.stdout, log
