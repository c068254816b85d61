"""Builds liblogmel.so in-tree for gfx950 with hipcc.

    python log_mel_spectrogram_amd/build.py

Steps: generate csrc/logmel_tables.h (fp64 math, fp32 literals), then one
hipcc invocation compiling the kernels and the C-ABI layer into a shared
library next to this file. All HIP code is compiled with packed-FP32
instruction selection disabled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblogmel.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("LOGMEL_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-fno-signed-zeros",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    subprocess.check_call([sys.executable, os.path.join(CSRC, "gen_tables.py"),
                           os.path.join(CSRC, "logmel_tables.h")])
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "logmel_kernels.hip"), os.path.join(CSRC, "logmel_resample.hip"),
           os.path.join(CSRC, "logmel_stream.hip"),
           os.path.join(CSRC, "logmel_static.hip"),
           os.path.join(CSRC, "logmel_api.cpp"),
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building liblogmel.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
