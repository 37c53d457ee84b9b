"""Build libpagedattn.so in-tree for gfx950.

Each HIP source is compiled with hipcc for gfx950 only; the host-only
allocator and status code are compiled with g++; everything is linked into
``paged_kv_cache_forward_amd/libpagedattn.so``.  Run ``python -m
paged_kv_cache_forward_amd.build`` (or call ``build()``).  ``--sanitize``
(``build_sanitized()``) instead builds the host allocator with the tests' trace
driver under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedattn.so")

HIP_SOURCES = ["cache_ops.hip", "decode.hip", "decode_mfma.hip", "decode_verify.hip", "decode_shared.hip",
               "prefill.hip", "forward.hip", "trace.hip"]
CXX_SOURCES = ["alloc.cpp", "status.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the device-only feature flag
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{res.stdout}\n{err}")
    return err


def build(verbose=False, extra_hip_flags=()):
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, *extra_hip_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in CXX_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for err in ex.map(_run, jobs):
            if verbose and err.strip():
                print(err, file=sys.stderr)
    objs = [os.path.join(OUT_DIR, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


# The host allocator under AddressSanitizer and UndefinedBehaviorSanitizer: the
# host-only sources (no GPU code) linked with the trace driver of the tests into
# one executable, built with g++.
SANITIZED_DRIVER = os.path.join(OUT_DIR, "alloc_driver_sanitized")
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=undefined", "-std=c++17", "-Wall", "-I" + INCLUDE, "-I" + CSRC]


def build_sanitized():
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = [os.path.join(ROOT, "tests", "alloc_driver.cpp")] + [os.path.join(CSRC, s) for s in CXX_SOURCES]
    tmp = SANITIZED_DRIVER + ".tmp"
    _run(["g++", *SANITIZE_FLAGS, *srcs, "-o", tmp])
    os.replace(tmp, SANITIZED_DRIVER)
    return SANITIZED_DRIVER


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build_sanitized())
    else:
        print(build(verbose=True))
