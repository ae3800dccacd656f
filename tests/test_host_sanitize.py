"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

falcon_api.cpp is rebuilt with the sanitizers on its host code only (its device
part, the allocation-free entry point's scratch array, is unchanged) and linked
with the kernel objects of the in-tree build into tests/host_sanitize_driver.cpp,
which calls every entry point of include/falcon.h with rejected and well-formed
arguments on a machine without a GPU (there every launch reports FALCON_ERR_HIP).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
CSRC = os.path.join(ROOT, "weight_recurrent_memory_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SKIP_EXIT = 77          # the driver's exit status where a GPU is present


def _kernel_objects():
    if not os.path.isdir(BUILD):
        return []
    return sorted(os.path.join(BUILD, f) for f in os.listdir(BUILD)
                  if f.endswith(".o") and not f.startswith("falcon_api"))


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), res.stdout[-3000:], res.stderr[-3000:])
    return res


def test_abi_layer_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC) or shutil.which("g++") is None:
        pytest.skip("hipcc or g++ not available")
    objs = _kernel_objects()
    if len(objs) < 9:
        pytest.skip("kernel objects not built (run __graft_entry__.build() first)")
    api = str(tmp_path / "api_asan.o")
    drv = str(tmp_path / "driver.o")
    exe = str(tmp_path / "driver")
    sanitize_host = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC] + sanitize_host
         + ["-Xarch_host", "-fno-omit-frame-pointer", "-x", "hip", "-c",
            os.path.join(CSRC, "falcon_api.cpp"), "-o", api])
    gxx_sanitize = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    _run(["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I" + INCLUDE] + gxx_sanitize
         + ["-c", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), "-o", drv])
    _run(["g++"] + gxx_sanitize + ["-o", exe, drv, api] + objs
         + ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = res.stdout + res.stderr
    if res.returncode == SKIP_EXIT:
        pytest.skip("a GPU is present: the driver's stand-in pointers are host memory")
    print(out[-2000:])
    assert "AddressSanitizer" not in out and "runtime error" not in out
    assert res.returncode == 0 and " 0 failures" in out
