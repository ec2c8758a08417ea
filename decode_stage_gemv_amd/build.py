"""Build libgrinqh.so (all HIP sources, gfx950) in place next to this file.

Usage: python -m decode_stage_gemv_amd.build [--timeline]

--timeline builds libgrinqh_timeline.so instead: the same library with the
VMM's clock stamps compiled in (grinqh_timeline_read), for measurement only.
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgrinqh.so")
# the same sources with the VMM's clock stamps compiled in (a measurement aid;
# see grinqh_timeline_read in include/grinqh.h)
LIB_TIMELINE = os.path.join(HERE, "libgrinqh_timeline.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # Keep the compiler from emitting packed fp32 arithmetic.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The leading scalar kernel arguments (up to twelve, as far as they fit
    # the user scalar registers; a structure argument ends the run) arrive
    # preloaded in scalar registers: the VMM kernels put every scalar their
    # prologues need there.  Without firmware support the kernel loads them
    # itself.
    "-mllvm", "-amdgpu-kernarg-preload-count=12",
    # Per-kernel register, scratch and occupancy report (checked below).
    "-Rpass-analysis=kernel-resource-usage",
]


def resource_usage(stderr: str) -> dict:
    """{kernel: {"VGPRs": n, "ScratchSize": n, "Occupancy": n}} from the compiler's remarks."""
    usage, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            usage[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            usage[name][m.group(1).split()[0]] = int(m.group(2))
    return usage


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Compile libgrinqh.so (or, with timeline=True, libgrinqh_timeline.so)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = LIB_TIMELINE if timeline else LIB
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *(["-DGRINQH_TIMELINE"] if timeline else []), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    usage = resource_usage(res.stderr)
    if not usage:
        raise RuntimeError("no kernel resource report from hipcc")
    # No kernel may spill to scratch (private memory): it turns register
    # arrays into slow memory round trips.  The VMM kernels must keep four
    # waves per SIMD (two 512-thread workgroups per CU).
    for name, u in usage.items():
        if u.get("ScratchSize", 0) != 0:
            raise RuntimeError(f"{name} uses {u['ScratchSize']} bytes of scratch per lane")
        if "vmm_kernel" in name and u.get("Occupancy", 0) < 4:
            raise RuntimeError(f"{name}: occupancy {u.get('Occupancy')} waves/SIMD, expected >= 4")
    if verbose:
        for name, u in sorted(usage.items()):
            print(f"  {name}: {u}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
