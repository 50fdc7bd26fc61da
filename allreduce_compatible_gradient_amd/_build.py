"""Build step of libgq.so: one hipcc invocation for gfx950 (MI355X)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", "gq.hip")]
LIB_PATH = os.path.join(PKG, "libgq.so")
# measurement kernels (read and VALU-issue ceilings), a library of their own
PROBE_SOURCES = [os.path.join(PKG, "csrc", "probe.hip")]
PROBE_LIB_PATH = os.path.join(PKG, "libgq_probe.so")

# -ffp-contract=off: every float operation rounds once, as the contract states.
# -fno-gpu-flush-denormals-to-zero: subnormal inputs are quantized, not flushed.
# -packed-fp32-ops off: no v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


# A compile normally takes well under a minute; a stalled compiler fails the
# build instead of blocking it.
BUILD_TIMEOUT_S = 900


def build_library(verbose: bool = False, sources=None, lib_path: str = LIB_PATH) -> str:
    sources = SOURCES if sources is None else sources
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources, "-o", tmp]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=BUILD_TIMEOUT_S)
    except subprocess.TimeoutExpired as e:
        raise RuntimeError(f"hipcc did not finish within {BUILD_TIMEOUT_S} s") from e
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, lib_path)
    return lib_path


def build_probe(verbose: bool = False) -> str:
    return build_library(verbose, PROBE_SOURCES, PROBE_LIB_PATH)


if __name__ == "__main__":
    print(build_library(verbose=True))
    print(build_probe(verbose=True))
