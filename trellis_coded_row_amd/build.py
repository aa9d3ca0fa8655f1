"""Builds the HIP libraries for gfx950 with hipcc, in-tree: libcp.so (the
lookup library, include/cp.h) and libcp_probe.so (measurement probes,
include/cp_probe.h)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "cp_decode.hip"), os.path.join(CSRC, "cp_dedup.hip"),
           os.path.join(CSRC, "cp_encode.hip"), os.path.join(CSRC, "cp_mixed.hip"),
           os.path.join(CSRC, "cp_shard.hip"), os.path.join(CSRC, "cp_dedup_mixed.hip"),
           os.path.join(CSRC, "cp_api.hip")]
DEPS = SOURCES + [os.path.join(CSRC, "cp_internal.h"), os.path.join(CSRC, "cp_lane.h"),
                  os.path.join(CSRC, "cp_encode_copies.h"),
                  os.path.join(ROOT, "include", "cp.h")]
LIB = os.path.join(PKG, "libcp.so")
PROBE_SOURCES = [os.path.join(CSRC, "cp_probe.hip")]
PROBE_LIB = os.path.join(PKG, "libcp_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 math: keep float code on plain (scalar-lane) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter", "-Wundef",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in DEPS)


def _hipcc(sources: list[str], lib: str, verbose: bool, extra_flags: list[str] | None) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"), *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Builds both libraries; returns the path of libcp.so."""
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose, extra_flags)
    return _hipcc(SOURCES, LIB, verbose, extra_flags)


if __name__ == "__main__":
    print(build(verbose=True))
