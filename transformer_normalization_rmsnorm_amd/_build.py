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
# kernel instances per storage type in units of their own, compiled in parallel
SOURCES = ["bwd_bf16.hip", "bwd_f32.hip", "bwd_f16.hip", "fwd_bf16.hip", "fwd_f32.hip", "fwd_f16.hip", "launch.hip",
           "api.cpp", "selector.cpp"]
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


def build(verbose: bool = False, resource_report: bool = True, jobs: int = 8) -> str:
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


FAMILIES = ("fwd_rows_kernel", "fwd_loop_kernel", "amax_finalize_kernel", "bwd_rows_kernel", "bwd_loop_kernel",
            "finalize_kernel")


def resource_summary(patterns=()) -> str:
    """Per-kernel resource usage of the last build (``_build/resource_usage.txt``):
    totals per kernel family, then every kernel whose demangled name contains
    one of `patterns` (bf16_t shown as bf16)."""
    path = os.path.join(BUILD, "resource_usage.txt")
    kernels, cur = [], None
    for ln in open(path):
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            cur = {"mangled": m.group(1)}
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?): (\d+)", ln)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    names = subprocess.run(["c++filt"], input="\n".join(k["mangled"] for k in kernels), capture_output=True,
                           text=True).stdout.splitlines()
    for k, n in zip(kernels, names):
        k["name"] = n.replace("rmsnorm::", "").replace("unsigned short", "bf16").replace("f16_t", "f16").replace("(rmsnorm::FwdArgs)", "") \
                     .replace("(rmsnorm::BwdArgs)", "").replace("(FwdArgs)", "").replace("(BwdArgs)", "")
    spilled = lambda k: k.get("VGPRs Spill", 0) or k.get("SGPRs Spill", 0) or k.get("ScratchSize [bytes/lane]", 0)
    out = [f"{'family':22s} {'kernels':>7s} {'max VGPRs':>9s} {'min occupancy':>13s} {'max LDS B':>9s} {'spilling':>8s}"]
    for fam in FAMILIES:
        ks = [k for k in kernels if re.search(r"\b" + fam + r"\b", k["name"])]
        if ks:
            out.append(f"{fam:22s} {len(ks):7d} {max(k.get('VGPRs', 0) for k in ks):9d} "
                       f"{min(k.get('Occupancy [waves/SIMD]', 0) for k in ks):13d} "
                       f"{max(k.get('LDS Size [bytes/block]', 0) for k in ks):9d} {sum(1 for k in ks if spilled(k)):8d}")
    out.append(f"{'all':22s} {len(kernels):7d} {'':9s} {'':13s} {'':9s} {sum(1 for k in kernels if spilled(k)):8d}")
    for pat in patterns:
        out.append("")
        out.append(f"kernels matching {pat!r}: VGPRs, SGPRs, occupancy (waves/SIMD), static LDS bytes, scratch bytes/lane")
        for k in kernels:
            if pat in k["name"]:
                out.append(f"  {k.get('VGPRs', 0):4d} {k.get('TotalSGPRs', 0):4d} {k.get('Occupancy [waves/SIMD]', 0):3d} "
                           f"{k.get('LDS Size [bytes/block]', 0):6d} {k.get('ScratchSize [bytes/lane]', 0):4d}  {k['name']}")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        if not os.path.exists(os.path.join(BUILD, "resource_usage.txt")):
            build()
        print(resource_summary(sys.argv[2:]))
    else:
        build(verbose=True)
    sys.exit(0)
