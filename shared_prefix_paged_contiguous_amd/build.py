"""Build libgkv.so in-tree with hipcc for gfx950.

    python -m shared_prefix_paged_contiguous_amd.build [--verbose]

One shared library holds the C ABI (include/gkv.h), the host planner and
allocators, and the HIP kernels.  It is built next to this file so that it
travels with the source tree.
"""

from __future__ import annotations

import argparse
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgkv.so")
SOURCES = ["kernels.hip", "gkv_api.cpp", "plan.cpp", "pools.cpp", "registry.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 VALU instructions (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no value is ever NaN (masked scores are -inf, which stays honoured), so
    # min/max need no NaN-quieting canonicalisation of MFMA results
    "-fno-honor-nans",
    "-Wall",
    "-Wno-unused-command-line-argument",
    # a kernel whose host stub went missing must fail the build, not the load
    "-Wl,-z,defs",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra=()) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgkv.so")
    if verbose and (res.stdout or res.stderr):
        sys.stderr.write(res.stdout + res.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def resource_usage() -> dict:
    """Per-kernel resource use of the device code, from the compiler's
    kernel-resource-usage remarks on a device-only compile of kernels.hip:
    {mangled kernel name: {"VGPRs": n, "AGPRs": n, "ScratchSize": bytes per
    lane, "VGPRs Spill": n, "SGPRs Spill": n, "Occupancy": waves per SIMD,
    "LDS Size": bytes per block, ...}}."""
    import re
    import tempfile
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc(), *[f for f in HIPCC_FLAGS if f not in ("-shared", "-Wl,-z,defs")],
               "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
               "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "kernels.hip"),
               "-o", os.path.join(tmp, "kernels.o")]
        res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed compiling kernels.hip")
    usage, name = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: +Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark: +([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+) \[", line)
        if m and name is not None:
            usage[name][m.group(1)] = int(m.group(2))
    return usage


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true",
                    help="print per-kernel VGPR/LDS/occupancy remarks")
    args = ap.parse_args()
    extra = ["-Rpass-analysis=kernel-resource-usage"] if args.resource_usage else []
    print(build(args.verbose or args.resource_usage, extra))


if __name__ == "__main__":
    main()
