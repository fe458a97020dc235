"""Build the native libraries in-tree.

* ``libsvattn.so``       - the C ABI (include/svattn.h): host core + HIP
  kernels for gfx950, built with hipcc.
* ``libsvattn_core.so``  - the HIP-free host core alone (include/svcore.h),
  built with g++, for host-logic tests on machines without a GPU.
* ``libsvattn_core_san.so`` - the same under ASan + UBSan with the verify
  planner's invariant checks compiled in (SVATTN_CHECKED).

Usage: ``python -m speculative_verify_attention_amd.build`` (or ``build()``).
Every call compiles from source; objects go to ``_build/`` beside the
package.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsvattn.so")
CORE_LIB = os.path.join(PKG, "libsvattn_core.so")
CORE_SAN_LIB = os.path.join(PKG, "libsvattn_core_san.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]

HIP_SOURCES = ["attn.hip", "attn_tq3.hip", "attn_valu.hip", "append.hip", "accept.hip", "probe.hip", "scratch.hip", "svattn.cpp",
               "kvcore.cpp", "plan.cpp", "ngram.cpp"]
CORE_SOURCES = ["kvcore.cpp", "plan.cpp", "svcore_capi.cpp", "ngram.cpp"]
# the host core again, under AddressSanitizer and UndefinedBehaviorSanitizer,
# with the planner's invariant checks compiled in (plain g++, no GPU code)
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-DSVATTN_CHECKED"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def _compile_hip(src, defines=(), tag=""):
    obj = os.path.join(BUILD, os.path.basename(src) + tag + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    _run([HIPCC, *HIP_FLAGS, *[f"-D{d}" for d in defines], *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build_core(sanitized=False):
    """libsvattn_core.so, or with sanitized=True libsvattn_core_san.so (load
    it with the sanitizer runtimes preloaded)."""
    os.makedirs(BUILD, exist_ok=True)
    out = CORE_SAN_LIB if sanitized else CORE_LIB
    flags = SAN_FLAGS if sanitized else ["-O2"]
    tmp = out + ".tmp"
    _run(["g++", *flags, "-std=c++17", "-fPIC", "-shared", "-Wall", "-I", INCLUDE, "-I", CSRC,
          *[os.path.join(CSRC, s) for s in CORE_SOURCES], "-o", tmp])
    os.replace(tmp, out)
    return out


def build_hip(jobs=None, out=LIB, defines=()):
    """Compile libsvattn.so; `defines` (NAME=VALUE) and `out` build a variant
    elsewhere without touching the in-tree library."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(4, os.cpu_count() or 1)
    tag = "" if not defines else "." + "_".join(d.replace("=", "") for d in defines)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile_hip(s, defines, tag), HIP_SOURCES))
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, out)
    return out


def build():
    core = build_core()
    build_core(sanitized=True)
    lib = build_hip()
    return lib, core


if __name__ == "__main__":
    for p in build():
        print(p)
    sys.exit(0)
