"""Build the HIP libraries in-tree with hipcc (gfx950 only).

Run ``python -m exact_tiled_attention_fa2_amd.build_lib`` or call ``build()``.
Two shared objects are built next to this file from the same sources:

* ``libattn_mi355x.so`` -- the release library the binding loads;
* ``libattn_mi355x_debug.so`` -- the same entry points plus those of
  ``include/attn_mi355x_debug.h`` (tile-shape overrides, per-row rescale
  counters and a matrix-core rate calibration), compiled with
  ``ATTN_DEBUG_BUILD`` (``attn_calib.hip`` compiles to nothing without it).

Each kernel source is compiled once per 16-bit type (``ATTN_TU_DTYPE``) so
that the translation units build in parallel.
"""

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
DEBUG_LIB_NAME = "libattn_mi355x_debug.so"
DEBUG_LIB_PATH = os.path.join(PKG_DIR, DEBUG_LIB_NAME)

# (source, extra defines) of one library; the kernel sources once per dtype.
UNITS = [("attn_kernels.hip", ["-DATTN_TU_DTYPE=0"]), ("attn_kernels.hip", ["-DATTN_TU_DTYPE=1"]),
         ("attn_bwd.hip", ["-DATTN_TU_DTYPE=0"]), ("attn_bwd.hip", ["-DATTN_TU_DTYPE=1"]),
         ("attn_api.cpp", []), ("attn_calib.hip", [])]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are kept out of the device code on purpose.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _clean(text):
    return "\n".join(line for line in text.splitlines()
                     if "is not a recognized feature for this target" not in line)


def _compile_jobs():
    """[(library path, objects, [(command, object)])] for both libraries."""
    libs = []
    for lib_path, extra in ((LIB_PATH, []), (DEBUG_LIB_PATH, ["-DATTN_DEBUG_BUILD=1"])):
        tag = "debug" if extra else "release"
        objs, jobs = [], []
        for src, defs in UNITS:
            suffix = "".join(d.split("=")[-1] for d in defs)
            obj = os.path.join(CSRC, "_build", tag, f"{src}{suffix}.o")
            cmd = [HIPCC, *COMMON_FLAGS, *extra, *defs]
            if src.endswith(".cpp"):
                cmd += ["-x", "hip"]
            cmd += [*DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
            objs.append(obj)
            jobs.append((cmd, obj))
        libs.append((lib_path, objs, jobs))
    return libs


def build(verbose=False, jobs=None):
    """Compile every unit of both libraries (in parallel) and link them; returns the release path."""
    jobs = jobs or max(1, min(16, os.cpu_count() or 4))
    libs = _compile_jobs()
    pending = [j for _, _, js in libs for j in js]
    running = []
    while pending or running:
        while pending and len(running) < jobs:
            cmd, obj = pending.pop(0)
            os.makedirs(os.path.dirname(obj), exist_ok=True)
            running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                  text=True)))
        cmd, proc = running.pop(0)
        out, _ = proc.communicate()
        if proc.returncode != 0:
            for _, other in running:
                other.kill()
            raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{_clean(out)}")
        if verbose and _clean(out).strip():
            print(_clean(out))
    for lib_path, objs, _ in libs:
        tmp = lib_path + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, "-o", tmp, *objs]
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{_clean(proc.stdout)}")
        os.replace(tmp, lib_path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
