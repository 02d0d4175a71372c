"""The host side of libqsa under AddressSanitizer and UndefinedBehaviorSanitizer:
the library's sources are compiled with both on the host pass only (the GPU
code is built as usual), linked with a C driver (tests/abi_sanitize_driver.c)
that makes every entry point reject bad arguments, run its zero-size no-ops
and size its workspace, and run on the CPU. A sanitizer report fails the test."""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparse_selection_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX) and shutil.which("gcc")),
                    reason="needs hipcc, ROCm's clang++ and gcc")
def test_host_library_is_clean_under_asan_and_ubsan(tmp_path):
    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-c",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC, src, "-o", obj]
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "driver.o")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, "abi_sanitize_driver.c"),
                    "-o", drv], check=True)
    exe = str(tmp_path / "abi_sanitize")
    subprocess.run([CLANGXX, "-fsanitize=address,undefined"] + objs + [drv, "-o", exe, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    # the HIP runtime keeps allocations for the life of the process: leak checks are off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "abi sanitizer driver: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
