"""Build libtsl.so: the gfx950 HIP kernels and the C ABI, in-tree.

Every translation unit is compiled by hipcc for gfx950 only; packed FP32
instructions are switched off for the device code (they are never needed
here).  Code objects are emitted as version 5 so that the HIP runtime a
PyTorch wheel carries (which may be older than this compiler) loads them.
Objects go to _build/ at the repository root.
"""
import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(PKG, "libtsl.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["abi.cpp", "plan.cpp", "pack.hip", "combine.hip", "embed.hip", "moe.hip", "skinny.hip", "prefill.hip", "q4gemm.hip",
           "noalloc.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-mcode-object-version=5", "-Wall",
         # only the C ABI of include/tsl.h is exported (it sets default visibility)
         "-fvisibility=hidden", "-fvisibility-inlines-hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the LDS-copy asm in prefill.hip sets m0 and lists it as clobbered on purpose
         "-Wno-inline-asm",
         "-I" + INCLUDE, "-I" + CSRC]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature name; that note is expected
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
    return obj, err


def exported_names():
    """The entry points include/tsl.h declares (its only exported names)."""
    with open(os.path.join(INCLUDE, "tsl.h")) as f:
        header = f.read()
    return re.findall(r"^(?:tsl_status|const char \*)\s*(\w+)\(", header, re.M)


def _version_script():
    path = os.path.join(OBJDIR, "tsl.map")
    body = "".join("    %s;\n" % n for n in exported_names())
    with open(path, "w") as f:
        # the HIP compiler's per-unit ids stay as they are emitted
        f.write("{\n  global:\n%s    __hip_cuid_*;\n  local: *;\n};\n" % body)
    return path


def build(verbose=False, jobs=None):
    """Compile all sources and link libtsl.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for obj, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    tmp = LIBRARY + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950",
           "-Wl,--version-script=" + _version_script(), "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
