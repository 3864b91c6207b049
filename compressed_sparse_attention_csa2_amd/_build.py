"""Build libcsa2.so (all HIP kernels + the C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
SOURCES = ["abi.hip", "compress.hip", "indexer.hip", "index_select.hip", "decode_select.hip",
           "attention.hip", "attention_dq.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # pinned operation order: no contraction of separate multiplies and adds
    "-ffp-contract=off",
    # keep fp32 denormals (the encoders see them as ordinary IEEE values)
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs (no accumulator-register copies in the epilogues)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


CALIB = os.path.join(HERE, "libcsa2calib.so")


def build_calib(verbose: bool = False) -> str:
    """the read-only streaming kernel the benchmark calibrates the decode scan with"""
    tmp = CALIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, os.path.join(CSRC, "calib.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libcsa2calib.so")
    os.replace(tmp, CALIB)
    return CALIB


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra or []), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libcsa2.so")
    if verbose and r.stderr.strip():
        # the host pass warns about the gfx-only target feature; keep other warnings visible
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized(out: str) -> str:
    """the library with its host code (argument checks, workspace layout, launch set-up)
    built with AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests of the
    checks that run before any launch; the device code is built as usual"""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    san = ["-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    cmd = [hipcc(), *HIPCC_FLAGS, *san, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs,
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building the host-sanitized library")
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_calib(verbose=True))
