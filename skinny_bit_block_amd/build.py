"""Build libqmm.so (the HIP library) in-tree with hipcc for gfx950."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmm.so")
SOURCES = ["qmm_kernels.hip", "qmm_api.cpp", "qmm_probe.hip", "gdn_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in l and "ignoring feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
