"""Builds libee.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree."""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libee.so")
SOURCES = [os.path.join(PKG, "csrc", n) for n in ("ee_api.hip", "ee_kernels.hip", "ee_proj.hip",
                                                      "ee_wide.hip", "ee_sample.hip", "ee_prefill.hip")]
# single-kernel launcher for hardware-counter runs (not part of the library)
PROBE = os.path.join(PKG, "ee_probe")
PROBE_SOURCES = [os.path.join(PKG, "csrc", n) for n in ("ee_probe.hip", "ee_proj.hip", "ee_wide.hip",
                                                          "ee_kernels.hip", "ee_prefill.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed float32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libee")
    return path


def _compile(out: str, sources, extra, verbose: bool):
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile libee.so (every kernel source and the C ABI) and the ee_probe
    launcher, in-tree; returns the library's path."""
    _compile(LIB, SOURCES, ["-shared"], verbose)
    _compile(PROBE, PROBE_SOURCES, [], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
