"""Build the test-only hardware probe library (tests/hw/libfa_probe.so) for
gfx950 with hipcc: the FP8 matrix-instruction probe, the XCD-assignment
probe and the instruction-issue-rate probe. Called by __graft_entry__.build(); the GPU tests that use it load the
built file and fail if it is missing."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libfa_probe.so")
SRCS = [os.path.join(HERE, f) for f in ("fp8_mfma_probe.hip", "xcd_probe.hip", "issue_probe.hip")]


def build() -> str:
    hipcc = next(c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
                 if c and os.path.exists(c))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-x", "hip", *SRCS,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {SRCS}:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
