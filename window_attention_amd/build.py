"""Build libwinattn.so (and the measurement library libwinprobe.so) in-tree
with hipcc for gfx950.

Run as ``python -m window_attention_amd.build``; ``__graft_entry__.build()``
calls ``build()``.  Every call recompiles from source.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
OBJ_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwinattn.so")
# measurement beside the path (bench.py's practical ceilings), a library of its own
PROBE_LIB = os.path.join(PKG, "libwinprobe.so")
PROBE_SOURCE = "mfma_probe.hip"
ARCH = "gfx950"

# packed fp32 VALU forms are switched off for all device code
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

SOURCES = [
    # the size formula's double arithmetic must not be contracted
    ("plan.hip", ["-ffp-contract=off"]),
    ("permute.hip", []),
    ("rope.hip", []),
    # MFMA results in VGPRs (the softmax reads every score: no AGPR copies);
    # no NaN quieting before each max (device code only: the host side of the
    # file validates arguments with isfinite)
    ("attn_fwd.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form", "-Xarch_device", "-fno-honor-nans"]),
    ("abi.cpp", ["-x", "hip"]),
    ("sp_plan.cpp", []),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    jobs = []
    for src, extra in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        jobs.append((obj, [hipcc, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *[j[0] for j in jobs], "-o", tmp])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc, *COMMON, "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
