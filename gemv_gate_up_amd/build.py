"""Builds libswiglu.so (the C-ABI library) in-tree with hipcc for gfx950, and
libswiglu_probe.so, bench.py's measurement aids.

Usage: python gemv_gate_up_amd/build.py   (or build() from Python; this file
is loaded by path so that it never imports the package, whose import needs
the built library)
"""
from __future__ import annotations

import concurrent.futures
import hashlib
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswiglu.so")
SOURCES = ["api.hip", "pack.hip", "skinny.hip", "wide.hip", "norm.hip", "fused.hip"]
# measurement aids for bench.py (a plain streaming read, device attributes),
# kept out of the library: their own shared object
PROBE_SRC = os.path.join(PKG, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(PKG, "libswiglu_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions are disabled for every device pass.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


# Per-kernel registers, LDS, occupancy, scratch and spills, printed by the
# compiler as analysis remarks (they do not change the generated code) and
# kept in RESOURCE_FILE for the tests.
REMARK_FLAGS = ["-Rpass-analysis=kernel-resource-usage"]
RESOURCE_FILE = os.path.join(OBJDIR, "resource_usage.json")
_REMARK = re.compile(r"remark:\s*([^:]+): (.*?) \[-Rpass-analysis=kernel-resource-usage\]")
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
           "ScratchSize [bytes/lane]": "scratch_bytes", "Dynamic Stack": "dynamic_stack",
           "Occupancy [waves/SIMD]": "occupancy", "SGPRs Spill": "sgpr_spill",
           "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds_bytes"}


def parse_resource_remarks(text: str) -> list:
    """One record per kernel from the compiler's resource-usage remarks."""
    kernels, cur = [], None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2).strip()
        if key == "Function Name":
            cur = {"kernel": val}
            kernels.append(cur)
        elif cur is not None and key in _FIELDS:
            cur[_FIELDS[key]] = (val == "True") if key == "Dynamic Stack" else int(val)
    return kernels


def source_fingerprint() -> str:
    """Hash of every library source and header the kernels are built from."""
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC)) + ["swiglu.h"]
    for f in files:
        path = os.path.join(CSRC if f != "swiglu.h" else INCLUDE, f)
        h.update(f.encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _compile(src: str):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + CFLAGS + REMARK_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    kernels = parse_resource_remarks(r.stderr)
    for k in kernels:
        k["source"] = src
    return obj, kernels


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    fingerprint = source_fingerprint()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    with open(RESOURCE_FILE, "w") as f:
        json.dump({"arch": ARCH, "sources": fingerprint,
                   "kernels": [k for _, ks in done for k in ks]}, f, indent=1)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + CFLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the probe library:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
