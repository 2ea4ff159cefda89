"""Build libsgemm.so (the HIP library) in-tree for gfx950 with hipcc.

    python -m chiplet_aware_persistent_amd.build [--jobs N]

Every translation unit under csrc/ is compiled to an object in parallel and
linked into chiplet_aware_persistent_amd/libsgemm.so.  Packed-fp32 instruction
selection is disabled for all device code.  The build fails if any kernel
uses scratch memory (SGEMM_ALLOW_SCRATCH=1 lets experiments through).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsgemm.so")
ARCH = os.environ.get("SGEMM_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I" + os.path.join(os.path.dirname(HERE), "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str):
    """Compile one translation unit; returns (object path, {kernel: scratch bytes per lane})."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr[-6000:]))
    static = {k: v for k, v in resource_usage(r.stderr, "LDS Size [bytes/block]").items()
              if v > STATIC_LDS_RESERVE}
    if static:
        raise RuntimeError("kernels declare more static LDS than the planner reserves (%d B): %s"
                           % (STATIC_LDS_RESERVE, static))
    return obj, scratch_usage(r.stderr)


def resource_usage(remarks: str, field: str) -> dict:
    """Per-kernel value of one field of the compiler's resource-usage remarks."""
    out, name = {}, None
    pat = re.compile(re.escape(field) + r": (\d+)")
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = pat.search(line)
        if m and name:
            out[name] = int(m.group(1))
    return out


def scratch_usage(remarks: str) -> dict:
    """Per-kernel private (scratch) bytes per lane."""
    return resource_usage(remarks, "ScratchSize [bytes/lane]")


# The planner keeps this much of the CU's 160 KB of LDS free for a kernel's
# static LDS (api.hip, kStaticLdsReserve).
STATIC_LDS_RESERVE = 256


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        res = list(ex.map(_compile, srcs))
    objs = [o for o, _ in res]
    # A kernel that spills (register pressure past 256 VGPRs, a dynamically
    # indexed array, a copy of the kernel arguments) runs several times slower
    # on this path; refuse to link one.
    spills = {k: v for _, u in res for k, v in u.items() if v > 0}
    if spills and not os.environ.get("SGEMM_ALLOW_SCRATCH"):
        raise RuntimeError("kernels use scratch memory (bytes per lane): %s" % spills)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr[-4000:]))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    a = ap.parse_args()
    try:
        build(a.jobs, verbose=True)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
