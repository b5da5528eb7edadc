"""The C ABI on the GPU from plain C: tests/c/abi_device (built by __graft_entry__.build() from
tests/c/abi_device.c with gcc, linked against libkvq.so and the HIP runtime, no PyTorch) appends
two tokens and decodes them; the program checks the outputs against their closed form."""

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_device")


@pytest.mark.gpu
def test_plain_c_client_on_gpu():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built (python -c 'import __graft_entry__ as g; g.build()')")
    print("[gpu] plain C client: append two tokens, decode", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FAIL" not in r.stdout and r.stdout.count("ok ") == 5
