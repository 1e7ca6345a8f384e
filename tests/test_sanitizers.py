"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (and the oracle's worker
threads under ThreadSanitizer), on the CPU.

- tests/sanitize/abi_host.cpp drives the library's C ABI: the host source (argument checks,
  sizing, error messages) is compiled here with the sanitizers, the kernel side comes from the
  built libkda.so and is never reached: every call is refused by validation or describes an
  empty problem.  Includes a seeded fuzz of kda_query / kda_chunk_bwd_workspace over edge-valued
  problem fields.
- tests/sanitize/oracle_host.c runs the C oracle on small odd-sized packed problems with every
  buffer at its exact size.

Only where no GPU is visible: the ABI driver passes fake device addresses, which only the
validation ever sees.
"""
import os
import shutil
import subprocess

import pytest

import gated_delta_rule_45_amd as kda
from gated_delta_rule_45_amd import build as kbuild

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(os.path.exists("/dev/kfd"),
                                reason="host-only sanitizer checks run where no GPU is visible")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=86",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87", TSAN_OPTIONS="exitcode=88")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not found")


def _build(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{res.stderr[-3000:]}"


def _run(exe, *args):
    res = subprocess.run([exe, *args], capture_output=True, text=True, env=ENV, timeout=300)
    out = res.stdout + res.stderr
    print(out[-2000:])
    assert "runtime error" not in out and "Sanitizer" not in out, out[-4000:]
    assert res.returncode == 0, f"exit {res.returncode}:\n{out[-4000:]}"
    assert " 0 failed" in out
    return out


def test_abi_host_code_under_asan_ubsan(tmp_path):
    _need("g++")
    kda.library()  # libkda.so must be built: it provides the kernel-side symbols
    exe = str(tmp_path / "abi_host")
    _build(["g++", "-std=c++17", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{kbuild.INCLUDE}",
            f"-I{kbuild.CSRC}", "-Wno-format-truncation", os.path.join(SAN, "abi_host.cpp"),
            os.path.join(kbuild.CSRC, "kda_api.cpp"), f"-L{kbuild.HERE}", f"-Wl,-rpath,{kbuild.HERE}", "-l:libkda.so",
            f"-L{ROCM}/lib", f"-Wl,-rpath,{ROCM}/lib", "-lamdhip64", "-o", exe])
    _run(exe, "20000")


def test_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_host")
    _build(["gcc", "-std=c11", *SAN_FLAGS, os.path.join(SAN, "oracle_host.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
            "-lpthread", "-lm", "-o", exe])
    _run(exe)


def test_oracle_threads_under_tsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_tsan")
    _build(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=thread", os.path.join(SAN, "oracle_host.c"),
            os.path.join(ROOT, "oracle", "kda_oracle.c"), "-lpthread", "-lm", "-o", exe])
    _run(exe)
