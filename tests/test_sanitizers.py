"""The host half of the library (C ABI size queries, parameter image,
argument checks) and the oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer and run on the CPU.  No GPU: the library's kernel
launchers and HIP runtime calls are stubbed in the driver
(tests/sanitize/host_abi_checks.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_decode_attention_quantize_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
CLANG = "/opt/rocm/llvm/bin/clang"


def _need(tool):
    if not os.path.exists(tool):
        pytest.skip(f"{tool} not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:]
    return r.stdout


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    return env


def test_host_abi_checks_under_sanitizers(tmp_path):
    _need(CLANG + "++")
    exe = str(tmp_path / "host_abi_checks")
    _run([CLANG + "++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "tq_host.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_abi_checks.cpp"),
          "-o", exe])
    out = _run([exe], env=_env())
    assert "host ABI checks clean" in out


def test_oracle_under_sanitizers(tmp_path):
    _need(CLANG)
    exe = str(tmp_path / "oracle_run")
    _run([CLANG, "-std=gnu99", *SAN, "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "oracle", "tq_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_run.c"),
          "-lm", "-o", exe])
    out = _run([exe], env=_env())
    assert "oracle run clean" in out
