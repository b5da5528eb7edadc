"""Build libkvq.so in-tree with hipcc for gfx950 (no torch involved)."""

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.hip", "quantize.hip", "decode_generic.hip", "decode_mfma.hip", "probes.hip",
           "tiering.hip", "prologue.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
    # keep MFMA accumulators in VGPRs: the online-softmax rescale touches them with VALU ops
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]
# The MFMA decoder assumes NaN-free inputs: without that, every maximum of DPP or cross-lane
# results gets an extra NaN-quieting instruction.
PER_FILE = {"decode_mfma.hip": ["-fno-honor-nans"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc, *FLAGS, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                text=True)))
            objs.append(obj)
        msgs = []
        failed = []
        for src, pr in procs:
            out, _ = pr.communicate()
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            msgs += lines
            if pr.returncode != 0:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for " + ", ".join(failed) + ":\n" + "\n".join(msgs))
        tmp_lib = LIB + ".tmp"
        rc, link_msgs = _run([hipcc, "--offload-arch=gfx950", "-fPIC", "-shared", "-fno-gpu-rdc",
                              *objs, "-o", tmp_lib])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(link_msgs))
        msgs += link_msgs
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
