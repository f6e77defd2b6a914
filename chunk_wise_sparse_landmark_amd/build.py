"""Compile the HiLS HIP library (libhils.so) and the input-fill helper for gfx950.

Every call recompiles.  Objects go to ``_build/`` next to this file; the shared
libraries are written in-tree (next to the Python modules that load them).
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops is switched off: the compiler then emits no packed fp32
# add/mul/fma instructions.
COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]

LIB = os.path.join(PKG, "libhils.so")
INPUTS_LIB = os.path.join(ROOT, "hils_inputs", "libhils_inputs.so")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    return out


def _link(objs, out):
    tmp = out + ".tmp"
    _run([HIPCC] + COMMON + ["-shared", "-o", tmp] + objs)
    os.replace(tmp, out)


def build(verbose=False, jobs=None):
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "hils_api.cpp")]
    jobs = jobs or min(8, os.cpu_count() or 4)

    def compile_one(src):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC] + COMMON + ["-I", INCLUDE, "-I", CSRC, "-c"] + lang + [src, "-o", obj])
        return obj

    fill_src = os.path.join(ROOT, "hils_inputs", "fill.hip")
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
        fill_obj = ex.submit(compile_one, fill_src).result()
    _link(objs, LIB)
    _link([fill_obj], INPUTS_LIB)
    if verbose:
        print("built", LIB, "and", INPUTS_LIB)
    return LIB


def clean():
    shutil.rmtree(os.path.join(PKG, "_build"), ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
