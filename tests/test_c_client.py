"""The C ABI from C: tests/c/abi_smoke.c includes include/flashblock.h as C99
(gcc -Wall -Werror), links libflashblock.so and checks version, workspace
size and validation paths on the CPU."""
import os
import shutil
import subprocess

import pytest

from cached_attention_amd import flashblock as fbl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c_client_compiles_links_and_validates(tmp_path):
    lib = fbl.lib()._name
    exe = tmp_path / "abi_smoke"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), lib, "-Wl,-rpath," + os.path.dirname(lib),
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_smoke ok" in r.stdout
