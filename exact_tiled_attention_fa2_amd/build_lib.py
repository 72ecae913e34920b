"""Build the HIP library libattn_mi355x.so in-tree with hipcc (gfx950 only).

Run ``python -m exact_tiled_attention_fa2_amd.build_lib`` or call ``build()``.
The host C++ and the kernels are compiled by hipcc into one shared object
next to this file; the Python binding loads it from there.
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
SOURCES = ["attn_kernels.hip", "attn_bwd.hip", "attn_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are kept out of the device code on purpose.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose=False, jobs=4):
    """Compile every source (in parallel) and link the shared library; returns its path."""
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src + ".o")
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [HIPCC, *COMMON_FLAGS, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        objs.append(obj)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    for cmd, proc in procs:
        out, _ = proc.communicate()
        if proc.returncode != 0:
            raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
