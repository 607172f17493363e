"""Build the HIP code in-tree for gfx950: libadamw4.so (the optimizer, C ABI in
include/adamw4.h), libadamw4_ceiling.so (a measurement kernel the benchmark runs beside the
step: the practical HBM ceiling for the step's byte mix) and hbm_mix_probe (a measurement
program: the byte mix's bandwidth under different access patterns, `bench.py --hbm-study`).

Flags: -ffp-contract=off keeps one rounding per FP32 operation in the code paths that decide
stored bits (clang-HIP's defaults already give correctly rounded division and square root and
keep FP32 denormals); packed-FP32 instructions are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libadamw4.so")
SOURCES = [os.path.join(CSRC, "adamw4_kernels.hip"), os.path.join(CSRC, "adamw4_api.cpp")]
CEILING_LIB = os.path.join(HERE, "libadamw4_ceiling.so")
CEILING_SOURCES = [os.path.join(CSRC, "stream_ceiling.hip")]
PROBE_EXE = os.path.join(HERE, "hbm_mix_probe")
PROBE_SOURCES = [os.path.join(CSRC, "hbm_mix_probe.hip")]
ARCH = os.environ.get("ADAMW4_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include")]


def _compile(out: str, sources: list[str], verbose: bool, shared: bool = True) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc()] + flags() + (["-shared"] if shared else []) + ["-o", tmp] + sources
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile libadamw4.so, libadamw4_ceiling.so and hbm_mix_probe (always recompiles)."""
    _compile(CEILING_LIB, CEILING_SOURCES, verbose)
    _compile(PROBE_EXE, PROBE_SOURCES, verbose, shared=False)
    return _compile(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
