"""Compile synth/libsynth.so (device input generator) with hipcc."""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "libsynth.so")


def build(verbose: bool = False) -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = OUT + ".tmp"
    cmd = [exe, "-x", "hip", "-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=gfx950",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "csrc", "synth.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on synth.hip:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
