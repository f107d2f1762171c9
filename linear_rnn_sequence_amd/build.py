"""Build librwkv7_wkv.so (HIP, gfx950) in-tree with hipcc.

Output: linear_rnn_sequence_amd/_lib/librwkv7_wkv.so
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIB_DIR, "librwkv7_wkv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the device compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA results in arch VGPRs (the chunked kernel feeds them straight back
    # into VALU conversions; AGPR results would add a copy per value)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = (["hipcc"] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC] + sources()
           + ["-o", tmp])
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build librwkv7_wkv.so")
    # the host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = ("packed-fp32-ops", "warning generated", "warnings generated")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if ln.strip()
            and not any(n in ln for n in noise)]
    if msgs and verbose:
        sys.stderr.write("\n".join(msgs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
