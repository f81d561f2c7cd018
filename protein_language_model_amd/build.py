"""Builds libesm_attn.so (HIP kernels + C ABI) in-tree for gfx950.

    python -m protein_language_model_amd.build [--verbose]

Each .hip source is compiled to an object in parallel under _build/, then
linked into protein_language_model_amd/libesm_attn.so; warnings are errors
(-Wall -Wextra -Werror). Packed-fp32 VALU
instructions are disabled for all device code (-packed-fp32-ops); the host
pass of hipcc warns that it does not know that feature, which is harmless.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libesm_attn.so")
SOURCES = ["api.hip", "prep.hip", "rope.hip", "fwd.hip", "bwd.hip", "batching.hip", "noalloc.hip",
           "merge.hip", "fwd_fp8.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
            "-Werror", "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "not a recognized feature" not in line)
    if p.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (p.returncode, " ".join(cmd), out))
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
