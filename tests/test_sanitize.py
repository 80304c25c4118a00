"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle's C (gcc) and the library's host code -- plans, sizes, the
validation that runs before any launch, the MoE dispatch -- (hipcc, the
sanitizers on the host side only; the kernels are compiled but never
launched) are built into two small drivers under tests/sanitize/, which
exercise them on small inputs and check the statuses the header promises;
any sanitizer report fails the run."""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tensor_sharded_linear_plan_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fopenmp", "-ffp-contract=off", "-o", exe,
         os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    r = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm")
def test_library_host_code_under_sanitizers(tmp_path):
    srcs = ["abi.cpp", "plan.cpp", "pack.hip", "combine.hip", "embed.hip", "moe.hip", "skinny.hip",
            "prefill.hip", "q4gemm.hip", "noalloc.hip"]
    flags = ["-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
             "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-inline-asm",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        run([HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-I" + os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "host_driver.cpp"),
         "-o", drv])
    exe = str(tmp_path / "host_driver")
    run([CLANG, "--hip-link", "--offload-arch=gfx950", "-fsanitize=address,undefined", "-o", exe,
         drv] + objs + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = run([exe], env=ENV)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr
