"""Compile the HIP sources under ``csrc/`` into ``libts.so`` (gfx950) and
the bounds-check variant ``libts_debug.so`` (the same sources compiled with
TS_DEBUG_CHECKS).

Usage: ``python -m convolution_voxelised_point_amd.build``.  hipcc
cross-compiles without a GPU.  Objects go to ``_build/`` (``_build_debug/``)
beside this file; the shared libraries land next to this file so the binding
finds them in-tree.
"""
from __future__ import annotations

import glob
import json
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libts.so")
DEBUG_BUILD_DIR = os.path.join(HERE, "_build_debug")
DEBUG_LIB = os.path.join(HERE, "libts_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions stay off: hipcc would otherwise form them from
# plain float code.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def cuid(src: str) -> str:
    """Fixed compilation-unit id of a source: it names the object's embedded
    GPU binary, so another host-side build of the same source (the sanitizer
    build of the tests) can link against that binary."""
    return "ts_" + os.path.splitext(os.path.basename(src))[0]


_REMARK = "-Rpass-analysis=kernel-resource-usage"
_FIELDS = {"VGPRs": "vgprs", "AGPRs": "agprs", "TotalSGPRs": "sgprs", "ScratchSize [bytes/lane]": "scratch_bytes",
           "Occupancy [waves/SIMD]": "waves_per_simd", "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text: str) -> dict:
    """Per-kernel register, scratch and LDS use from the compiler's
    kernel-resource-usage remarks: {mangled name: {field: int}}."""
    out, cur = {}, None
    for line in text.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].replace("[" + _REMARK + "]", "").strip()
        if body.startswith("Function Name:"):
            cur = out.setdefault(body.split(":", 1)[1].strip(), {})
            continue
        m = re.match(r"(.+?):\s*(-?\d+)$", body)
        if cur is not None and m and m.group(1) in _FIELDS:
            cur[_FIELDS[m.group(1)]] = int(m.group(2))
    return out


def resources_path(src: str) -> str:
    return os.path.join(BUILD_DIR, os.path.basename(src) + ".resources.json")


def _compile(src: str, debug: bool = False) -> str:
    """Compiles one source; the regular build also writes the kernels'
    resource use (registers, scratch, LDS) beside the object."""
    obj = os.path.join(DEBUG_BUILD_DIR if debug else BUILD_DIR, os.path.basename(src) + ".o")
    extra = ["-DTS_DEBUG_CHECKS"] if debug else [_REMARK]
    cmd = [HIPCC, *CFLAGS, *extra, f"-cuid={cuid(src)}", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    if not debug:
        with open(resources_path(src), "w") as f:
            json.dump(parse_resource_remarks(r.stderr), f, indent=0, sort_keys=True)
    noise = "is not a recognized feature for this target"
    kept, in_remark = [], False
    for line in r.stderr.splitlines():
        if ": remark:" in line:
            in_remark = True  # a remark and the source excerpt under it
        elif ": warning:" in line or ": error:" in line or ": note:" in line:
            in_remark = False
        if not in_remark and noise not in line:
            kept.append(line)
    errs = "\n".join(kept)
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def link(objs, lib: str) -> str:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(jobs: int = 8, debug: bool = True) -> str:
    """Builds libts.so and, with `debug`, libts_debug.so; returns the path
    of libts.so."""
    variants = [False, True] if debug else [False]
    for d in variants:
        os.makedirs(DEBUG_BUILD_DIR if d else BUILD_DIR, exist_ok=True)
    jobs_list = [(src, d) for d in variants for src in sources()]
    # the slowest sources first, so the pool ends together
    jobs_list.sort(key=lambda j: -os.path.getsize(j[0]))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda j: (j[1], _compile(*j)), jobs_list))
    for d in variants:
        link(sorted(o for dd, o in objs if dd == d), DEBUG_LIB if d else LIB)
    return LIB


if __name__ == "__main__":
    print(build())
