"""Sanitizer builds of the native CPU code (no GPU needed).

* The oracle (oracle/oracle.c) is built by gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer, and the oracle's whole test module (every pin,
  and the 26 planted-mistake checks, whose mutants are built without
  sanitizers: a planted mistake that reads out of bounds fails its pin, or
  here would stop the run) runs against it in a child process with the
  sanitizer runtime preloaded.
* The host side of the HIP library (argument validation, partition and
  schedule planning, workspace sizing, the C entry points up to the launch)
  is compiled host-only by hipcc with the same sanitizers, linked with an
  empty stand-in for the device code object (nothing here launches a
  kernel), and the C-ABI tests run against it.

Any sanitizer report ends the child with an error and fails the test. Both
builds go to a temporary directory; the in-tree libraries are not touched.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0", "UBSAN_OPTIONS": "print_stacktrace=1"}


def run_child(tests, env_extra, tmp_path):
    env = dict(os.environ, **SAN_ENV, **env_extra)
    cmd = [sys.executable, "-m", "pytest", *tests, "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    log = res.stdout + res.stderr
    (tmp_path / "child.log").write_text(log)
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-4000:]
    assert res.returncode == 0, log[-4000:]
    return log


def test_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    so = tmp_path / "liboracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
                    "-pthread", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", str(so), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    log = run_child(["tests/test_oracle.py"], {"LD_PRELOAD": asan, "ORACLE_LIB": str(so)}, tmp_path)
    assert re.search(r"\d+ passed", log)


def asan_runtime():
    res = subprocess.run([HIPCC, "-print-resource-dir"], capture_output=True, text=True)
    path = os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
    return path if os.path.exists(path) else None


def test_library_host_side_under_asan_and_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    rt = asan_runtime()
    if rt is None:
        pytest.skip("the compiler's AddressSanitizer runtime was not found")
    obj = tmp_path / "mqa_host.o"
    src = os.path.join(ROOT, "transformer_decode_attention_amd", "csrc", "mqa_decode.hip")
    # host-only: the device pass is not run (the sanitizers apply to host code only)
    flags = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Wall", "-Werror", "-Wno-unused-command-line-argument",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
             "-I", os.path.join(ROOT, "include")]
    res = subprocess.run([HIPCC, *flags, "-c", "-o", str(obj), src], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    # the code object the host part registers at load: an empty stand-in
    nm = subprocess.run(["nm", "-u", str(obj)], capture_output=True, text=True, check=True).stdout
    syms = sorted(set(re.findall(r"__hip_fatbin_[0-9a-f]+", nm)))
    stub = tmp_path / "stub.c"
    stub.write_text("".join(f"const char {s}[64] = {{0}};\n" for s in syms))
    subprocess.run(["gcc", "-c", "-fPIC", "-o", str(tmp_path / "stub.o"), str(stub)], check=True)
    so = tmp_path / "libmqa_san.so"
    res = subprocess.run([HIPCC, "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                          "-Xarch_host", "-fsanitize=undefined", "-o", str(so), str(obj),
                          str(tmp_path / "stub.o")], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    log = run_child(["tests/test_abi.py", "tests/test_abi_properties.py"],
                    {"LD_PRELOAD": rt, "MQA_DECODE_LIB": str(so)}, tmp_path)
    assert re.search(r"\d+ passed", log)
