"""Ahead-of-time build of libcsa.so for gfx950 with hipcc (no JIT).

    python -m sparse_compressed_attention_amd.build

writes sparse_compressed_attention_amd/libcsa.so next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libcsa.so")
SOURCES = ["index_scores.hip", "topk.hip", "attn.hip", "csa_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsa.so)")


def build_command(out_path: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed FP32 VALU ops are kept off for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out_path,
    ]


C_DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi", "decode_step.cpp")
C_DRIVER = os.path.join(ROOT, "tests", "c_abi", "decode_step")


def build_c_driver(verbose: bool = False) -> str:
    """The test driver that runs a decode step through the C ABI alone
    (linked against libcsa.so next to this file)."""
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", INCLUDE, C_DRIVER_SRC, "-L", PKG_DIR, "-lcsa",
           "-Wl,-rpath,$ORIGIN/../../sparse_compressed_attention_amd", "-o", C_DRIVER]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return C_DRIVER


PEAK_LIB_PATH = os.path.join(PKG_DIR, "libcsa_peak.so")


def peak_build_command(out_path: str) -> list[str]:
    """The benchmark's peak probes (plain copy, FP8 MFMA loop): a library of
    their own, never loaded by the CSA path."""
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        os.path.join(CSRC, "peak.hip"), "-o", out_path,
    ]


def _build_lib(make_cmd, dest: str, verbose: bool) -> None:
    fd, tmp = tempfile.mkstemp(prefix="." + os.path.basename(dest) + ".", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    try:
        cmd = make_cmd(tmp)
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
        os.replace(tmp, dest)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)


def build(verbose: bool = False) -> str:
    _build_lib(build_command, LIB_PATH, verbose)
    _build_lib(peak_build_command, PEAK_LIB_PATH, verbose)
    build_c_driver(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
