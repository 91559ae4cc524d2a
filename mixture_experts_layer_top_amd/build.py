"""Builds libmoe_mi355x.so in-tree with hipcc for gfx950 (host-side cross-compile; no GPU needed).

    python -m mixture_experts_layer_top_amd.build
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_mi355x.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Device code: gfx950 only; packed fp32 ops disabled (the host pass warns that it does not know
# the feature, which is harmless).
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


# Every kernel must keep its registers: the compiler's resource-usage remarks are read back and a
# kernel that spills to scratch memory fails the build.
RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"


def kernel_resources(remarks: str) -> dict[str, dict[str, str]]:
    """Per-kernel fields of the compiler's kernel-resource-usage remarks (VGPRs, AGPRs,
    ScratchSize [bytes/lane], Occupancy [waves/SIMD], ...)."""
    out: dict[str, dict[str, str]] = {}
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark: (.*?) \[-Rpass-analysis=kernel-resource-usage\]", line)
        if not m:
            continue
        key, _, val = m.group(1).partition(":")
        if key.strip() == "Function Name":
            cur = out.setdefault(val.strip(), {})
        elif cur is not None:
            cur[key.strip()] = val.strip()
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, *HIP_FLAGS, *COMMON, RESOURCE_REMARKS, "-x", "hip", "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if src.endswith(".hip"):
        res = kernel_resources(r.stderr)
        with open(obj + ".resources.txt", "w") as fh:
            for name, f in sorted(res.items()):
                fh.write(f"{name}: " + ", ".join(f"{k}={v}" for k, v in f.items()) + "\n")
        spills = {n: f.get("ScratchSize [bytes/lane]") for n, f in res.items()
                  if f.get("ScratchSize [bytes/lane]", "0") != "0"}
        if spills:
            raise RuntimeError(f"{os.path.basename(src)}: kernels use scratch memory (register "
                               f"spills), bytes per lane: {spills}")
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source (always, so the result matches the tree) and links the library."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
