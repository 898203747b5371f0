"""Build libfa.so (the gfx950 attention kernels + C ABI) in-tree with hipcc.

Usage: python -m exact_attention_27_amd.build [--verbose]

Always recompiles. The library lands next to this file as ``libfa.so``; the compiler's
per-kernel resource report (VGPR/AGPR/SGPR, LDS, spills, occupancy) is written to
``kernel_resources.txt`` beside it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfa.so")
RESOURCES = os.path.join(HERE, "kernel_resources.txt")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libfa.so")


# Per-source extra flags. MFMA results go to VGPRs: the kernels feed S and dP straight to
# VALU softmax code, and AGPR-destination MFMAs made the allocator shuttle accumulators
# between the two register files on every loop iteration.
VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCES = {
    "fa_api.cpp": [],
    "fa_fwd.hip": VGPR_FORM,
    "fa_bwd.hip": VGPR_FORM,
    "fa_bwd_dkv.hip": VGPR_FORM,
    # 256-wide dK/dV: more registers than the VGPR form can hold (see the file's header)
    "fa_bwd_dkv_wide.hip": [],
    # the backward entry point whose workspace is a static device array (no allocation)
    "fa_noalloc.hip": [],
}


def _common(cc):
    return [
        cc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-function",
        # Keep the compiler from forming packed fp32 VALU instructions.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(os.path.dirname(HERE), "include"),
    ]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    report, other, objs = [], [], []
    # one compiler process per unit, all at once (at most len(SOURCES), a handful)
    procs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(objdir, src + ".o")
        cmd = _common(cc) + extra + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                      os.path.join(CSRC, src), "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    failed = None
    for src, obj, proc in procs:
        _, err = proc.communicate()
        report += [ln for ln in err.splitlines() if "remark:" in ln]
        other += [ln for ln in err.splitlines()
                  if "remark:" not in ln and "packed-fp32-ops" not in ln and ln.strip()]
        if proc.returncode != 0 and failed is None:
            failed = (src, proc.returncode)
        objs.append(obj)
    if failed is not None:
        sys.stderr.write("\n".join(other) + "\n")
        raise RuntimeError(f"hipcc failed on {failed[0]} with exit code {failed[1]}")
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp"] + objs
    proc = subprocess.run(link, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stderr)
        raise RuntimeError(f"link failed with exit code {proc.returncode}")
    os.replace(LIB + ".tmp", LIB)
    with open(RESOURCES, "w") as f:
        f.write("\n".join(_condense(report)) + "\n")
    if verbose and other:
        sys.stderr.write("\n".join(other) + "\n")
    return LIB


def _condense(lines):
    out = []
    for ln in lines:
        msg = ln.split("remark:", 1)[1].strip()
        out.append(msg.replace(" [-Rpass-analysis=kernel-resource-usage]", ""))
    return out


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
