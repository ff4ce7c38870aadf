"""Host sanitizer runs (no GPU): the CPU oracle and the C-ABI argument checks,
built with AddressSanitizer and UndefinedBehaviorSanitizer and driven over
every entry point (tests/sanitize/*.c*).  The ABI build replaces the kernel
launchers with stubs, so the checks of maskgs_api.hip run for real on
arguments that name fake, aligned device addresses."""
import os
import shutil
import subprocess

import pytest

from conftest import REPO

SAN = os.path.join(REPO, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")


def _run(exe, tmp_path, leaks=True):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = f"detect_leaks={1 if leaks else 0}:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env, cwd=tmp_path)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "orc_san")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-ffp-contract=off",
           os.path.join(SAN, "oracle_driver.c"), os.path.join(REPO, "oracle", "maskgs_oracle.c"),
           os.path.join(REPO, "oracle", "maskpro_oracle.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    _run(exe, tmp_path)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_san")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]
    csrc = os.path.join(REPO, "sparsity_masks_weights_amd", "csrc")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_san,
           "-I", os.path.join(REPO, "include"), "-I", csrc,
           os.path.join(csrc, "maskgs_api.hip"), os.path.join(SAN, "abi_stubs.cpp"),
           os.path.join(SAN, "abi_driver.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=900)
    _run(exe, tmp_path)
