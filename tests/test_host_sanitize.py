"""The host layer of the library (fb_api.cpp: validation, split planning,
launch arguments) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, linked with host-only stand-ins of the kernel
launchers (tests/c/launch_stubs.cpp), and driven on the CPU through every
entry point over the workload shapes and the size limits
(tests/c/host_paths.c).  No GPU and no HIP runtime are involved: the stand-ins
check each launch's work-item count and grid instead of launching."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
INC = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "cached_attention_amd", "csrc")]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="gcc/g++ not available")
def test_host_layer_under_asan_ubsan(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    objs = []
    for src in (os.path.join(ROOT, "cached_attention_amd", "csrc", "fb_api.cpp"),
                os.path.join(ROOT, "tests", "c", "launch_stubs.cpp")):
        obj = tmp_path / (os.path.basename(src) + ".o")
        r = subprocess.run(["g++", "-std=c++17", "-Wall", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", f"{rocm}/include",
                            *INC, "-c", src, "-o", str(obj)], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(str(obj))
    obj = tmp_path / "host_paths.o"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", *SAN, *INC, "-c",
                        os.path.join(ROOT, "tests", "c", "host_paths.c"), "-o", str(obj)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "host_paths"
    r = subprocess.run(["g++", *SAN, *objs, str(obj), "-o", str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("FB_DEBUG", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host_paths ok" in r.stdout
