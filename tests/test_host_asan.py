"""Host entry points under AddressSanitizer (CPU).

Builds the host-side planner, packing, SP-table and rotary-table code with
AddressSanitizer on the host compilation only (device code is untouched), links
it with tests/asan/host_driver.cpp, and runs the driver: it sweeps grids,
window counts, both methods, rank counts and packing alignments with every
table allocated at exactly its documented size, so any read or write past a
table aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "window_attention_amd", "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "asan")


def _tool(name, fallback):
    path = shutil.which(name) or fallback
    return path if path and os.path.exists(path) else None


HIPCC = _tool("hipcc", "/opt/rocm/bin/hipcc")
GXX = _tool("g++", None)


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(HIPCC is None or GXX is None, reason="needs hipcc and g++")
def test_host_entry_points_under_asan():
    os.makedirs(OUT, exist_ok=True)
    hip = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           f"-I{CSRC}", f"-I{INC}"]
    cxx = [GXX, "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address", "-fno-omit-frame-pointer", f"-I{CSRC}",
           f"-I{INC}"]
    objs = []
    for src in ("plan.hip", "rope.hip", "abi.cpp"):
        obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
        _run(hip + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src, obj in ((os.path.join(CSRC, "sp_plan.cpp"), "sp_plan.o"),
                     (os.path.join(ROOT, "tests", "asan", "host_driver.cpp"), "driver.o")):
        _run(cxx + ["-c", src, "-o", os.path.join(OUT, obj)])
        objs.append(os.path.join(OUT, obj))
    exe = os.path.join(OUT, "host_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "AddressSanitizer" not in r.stdout, r.stdout[-4000:]
    assert r.stdout.strip().startswith("ok "), r.stdout[-2000:]
    assert int(r.stdout.split()[1]) > 1000  # every sweep point ran
