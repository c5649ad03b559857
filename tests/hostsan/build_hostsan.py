"""Build the C-ABI layer for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer (g++), kernel launchers stubbed out:
tests/hostsan/_build/libfa_hostsan.so. Used by
tests/test_abi_host_sanitized.py, which runs the ABI tests against it."""

from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "exact_attention_120_amd", "csrc")
OUT = os.path.join(HERE, "_build", "libfa_hostsan.so")
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer"]


def compiler() -> str | None:
    return shutil.which("g++")


def runtime_library() -> str | None:
    """The ASan runtime g++ links against (it must be loaded first)."""
    gxx = compiler()
    if not gxx:
        return None
    res = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    return os.path.realpath(path) if res.returncode == 0 and os.path.isabs(path) \
        and os.path.exists(path) else None


def _compile(srcs: list[str], out: str) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [compiler(), "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Werror"] \
        + SANITIZE + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                      "-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + ["-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("host sanitizer build failed:\n" + res.stderr)
    return out


def build() -> str:
    return _compile([os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_host.cpp"),
                     os.path.join(HERE, "stub_launch.cpp")], OUT)


def build_planted() -> str:
    """The planted-mistake library (planted_oob.cpp), same flags."""
    return _compile([os.path.join(HERE, "planted_oob.cpp")],
                    os.path.join(HERE, "_build", "libplanted.so"))


if __name__ == "__main__":
    print(build())
