"""Build liblwo.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python layerwise_weight_offload_amd/build.py

(run it as a script: importing the package would load the library it is
about to replace).

Every source under csrc/ is compiled with hipcc for gfx950 only; packed fp32
VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblwo.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["layout.cpp", "store.cpp", "cache.cpp", "ops.cpp", "block.hip", "k_rows.hip", "k_gemm.hip", "k_attn.hip", "k_attn_f32.hip", "k_probe.hip",
           "noalloc.hip"]

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# Kernels that read LDS with inline asm and await the reads with explicit
# lgkmcnt waits: the compiler treats an asm output as written when the asm is
# issued, so a spill of such a register between the read and its wait would
# store a value that has not arrived yet.  They must not use scratch, and the
# build fails if one does.
NO_SCRATCH = ("k_gemm_deep", "k_attn_tr")


def _scratch_users(remarks: str) -> list[str]:
    """Kernels of NO_SCRATCH whose resource-usage remark reports scratch."""
    bad, fn = [], None
    for ln in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", ln)
        if m:
            fn = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", ln)
        if m and fn and int(m.group(1)) > 0 and any(k in fn for k in NO_SCRATCH):
            bad.append(f"{fn} ({m.group(1)} bytes/lane)")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    bad = _scratch_users(r.stderr)
    if bad:
        raise RuntimeError(f"{src}: kernels with inline-asm LDS reads use scratch: " + ", ".join(bad))
    noise = ("is not a recognized feature for this target", "remark: ", "-Rpass-analysis")
    keep = []
    for ln in r.stderr.splitlines():
        if any(n in ln for n in noise):
            continue
        keep.append(ln)
    # drop the source excerpts that belonged to the filtered remarks
    err = "\n".join(ln for ln in keep if "warning" in ln or "error" in ln)
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
