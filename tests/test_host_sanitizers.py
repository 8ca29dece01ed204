"""The host packer (decode_gemv_tensor_amd/csrc/host_pack.cpp) and the oracle
(oracle/binade_oracle.c) built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++/gcc, CPU only) and run over many shapes, all
bf16 patterns, exact-size buffers, too-small buffers and corrupt streams. The
two are built as separate programs: they share no code."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "unrecognized" in r.stderr:
        pytest.skip("compiler without sanitizer support")
    assert r.returncode == 0, r.stderr[-3000:]
    env = {**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
           "UBSAN_OPTIONS": "print_stacktrace=1"}
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_host_packer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "host_pack_san")
    cmd = ["g++", "-std=c++17"] + SAN + [
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "decode_gemv_tensor_amd", "csrc"),
        os.path.join(HERE, "host_pack_driver.cpp"),
        os.path.join(ROOT, "decode_gemv_tensor_amd", "csrc", "host_pack.cpp"), "-o", exe]
    assert "host packer: ok" in _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    cmd = ["gcc", "-std=c99", "-ffp-contract=off"] + SAN + [
        os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "binade_oracle.c"),
        "-lm", "-o", exe]
    assert "oracle: ok" in _build_and_run(cmd, exe)
