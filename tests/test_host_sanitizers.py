"""AddressSanitizer + UndefinedBehaviorSanitizer over the library's host code.

The host logic of the C ABI (argument validation, workspace and plan sizes,
the cu_seqlens checker, the schedule model, the length-bucketing batcher)
lives in api.hip and batching.hip. Both are compiled host-only with the
sanitizers on the host pass, linked with the kernel objects of the normal
build (their host side is only launch code), and driven by host_driver.cpp,
which calls every host-only entry point and every validation path on fixed
and seeded random inputs and checks their invariants. No GPU is used.
"""

import os
import subprocess

import pytest

from protein_language_model_amd import build as B

KERNEL_SOURCES = [s for s in B.SOURCES if s not in ("api.hip", "batching.hip")]
HERE = os.path.dirname(os.path.abspath(__file__))

# each sanitizer flag goes to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined"]


def _kernel_objects():
    """Objects of the normal build, rebuilt if missing or older than a source."""
    objs = [os.path.join(B.BUILD, s.replace(".hip", ".o")) for s in KERNEL_SOURCES]
    srcs = [os.path.join(dr, f) for dr in (B.CSRC, B.INCLUDE) for f in os.listdir(dr)]
    newest = max(os.path.getmtime(p) for p in srcs)
    if not all(os.path.exists(o) and os.path.getmtime(o) >= newest for o in objs):
        B.build()
    return objs


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    assert p.returncode == 0, "%s\n%s" % (" ".join(cmd), p.stdout[-4000:])
    return p.stdout


def test_host_code_under_sanitizers(tmp_path):
    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    common = ["--offload-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
              "-fno-omit-frame-pointer", "-Wall", "-Werror", "-Wno-unused-function",
              "-I", B.INCLUDE, "-I", B.CSRC] + SAN
    host_objs = []
    for src in (os.path.join(B.CSRC, "api.hip"), os.path.join(B.CSRC, "batching.hip"),
                os.path.join(HERE, "host_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([cc] + common + ["-c", src, "-o", obj])
        host_objs.append(obj)
    exe = str(tmp_path / "host_driver")
    _run([cc] + SAN + ["-o", exe] + host_objs + _kernel_objects())
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=300, env=env)
    assert p.returncode == 0 and "host driver ok" in p.stdout, p.stdout[-4000:]
    assert "runtime error" not in p.stdout and "AddressSanitizer" not in p.stdout, p.stdout
