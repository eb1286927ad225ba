"""The CPU oracle and the library's host-side packer built with gcc under AddressSanitizer and
UndefinedBehaviorSanitizer, and exercised by tests/sanitize/host_driver.c (packers on ragged
shapes, the stacked and gate / up layouts with their in-place moves, the rotated packing, and
the oracle's forward paths).  CPU only: nothing here touches a GPU."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="gcc needed")
def test_oracle_and_host_packer_under_asan_ubsan(tmp_path):
    inc = os.path.join(ROOT, "include")
    objs = []
    steps = [
        ["gcc", "-std=c11", "-ffp-contract=off", "-c", os.path.join(ROOT, "oracle", "bitnet_oracle.c"),
         "-o", str(tmp_path / "oracle.o")],
        ["g++", "-std=c++17", "-c", os.path.join(ROOT, "ternary_weight_bit_bitlinear_amd", "csrc", "pack_host.cpp"),
         "-I", inc, "-o", str(tmp_path / "pack_host.o")],
        ["gcc", "-std=c11", "-c", os.path.join(ROOT, "tests", "sanitize", "host_driver.c"), "-I", inc,
         "-o", str(tmp_path / "driver.o")],
    ]
    for cmd in steps:
        cmd[1:1] = SAN
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        objs.append(cmd[cmd.index("-o") + 1])
    exe = str(tmp_path / "host_driver")
    subprocess.run(["g++"] + SAN + objs + ["-o", exe, "-lm"], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host driver ok" in r.stdout
