"""Ahead-of-time build of the gfx950 RMSNorm library with hipcc (no JIT).

``python -m transformer_normalization_rmsnorm_amd._build`` compiles every
source in ``csrc/`` for gfx950 and links ``librmsnorm_amd.so`` in this package
directory.  The kernel resource usage (VGPRs, SGPRs, LDS, scratch) reported by
the compiler is kept in ``_build/resource_usage.txt``.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBRARY = os.path.join(PKG, "librmsnorm_amd.so")
SOURCES = ["api.cpp", "selector.cpp", "fwd_kernels.hip", "bwd_kernels.hip"]
# measurement-only library (practical bandwidth ceilings for the benchmark)
PROBE_SOURCE = "stream_probe.hip"
PROBE_LIBRARY = os.path.join(PKG, "libstream_probe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed-f32 instructions are generated (they are avoided on this part)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str, resource_report: bool) -> tuple:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + CFLAGS
    if resource_report and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj, r.stderr


def build(verbose: bool = False, resource_report: bool = True, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_report), SOURCES))
    objs = [o for o, _ in results]
    report = "".join(err for _, err in results)
    usage = [ln for ln in report.splitlines() if "remark:" in ln and not ln.endswith("warning")]
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write("\n".join(usage) + "\n")
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIBRARY)
    tmp = PROBE_LIBRARY + ".tmp"
    cmd = [HIPCC, "-x", "hip", "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp] + CFLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SOURCE}:\n{r.stderr[-4000:]}")
    os.replace(tmp, PROBE_LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
        spills = [ln for ln in usage if re.search(r"(ScratchSize|Spill)\S*: [1-9]", ln)]
        if spills:
            print("kernels with scratch or spills:\n" + "\n".join(spills[:20]))
    return LIBRARY


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
