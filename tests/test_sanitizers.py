"""AddressSanitizer and UBSan over the CPU-side code (CPU only, no GPU call):
the oracle, run on small inputs of every entry (tests/sanitize/oracle_driver.c,
built with gcc), and the library's host-side argument checks and workspace
queries (tests/sanitize/abi_driver.cpp, built from the library's own source
with the sanitizers on its host code only).  The second build takes about a
minute and a half; it is kept under tests/sanitize/_build/ by source hash."""
import hashlib
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
BUILD = os.path.join(SAN, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CSRC = os.path.join(ROOT, "moe_expert_dequant_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    src = [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    flags = ["-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-ffp-contract=off"]
    exe = os.path.join(BUILD, "oracle_san_" + digest(src + [os.path.join(ROOT, "oracle", "oracle.h")], flags))
    if not os.path.exists(exe):
        subprocess.run(["gcc"] + flags + ["-I", os.path.join(ROOT, "oracle")] + src + ["-lm", "-o", exe],
                       check=True, capture_output=True, timeout=300)
    assert "ok" in run(exe)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_host_under_asan_ubsan():
    os.makedirs(BUILD, exist_ok=True)
    hdrs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    src = [os.path.join(CSRC, "ffnq.hip"), os.path.join(SAN, "abi_driver.cpp")]
    # the sanitizers instrument the host code only (each -fsanitize= right after -Xarch_host)
    flags = ["--offload-arch=gfx950", "-O1", "-fno-omit-frame-pointer", "-std=c++17", "-Xarch_host", "-g",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    exe = os.path.join(BUILD, "abi_san_" + digest(src + hdrs + [os.path.join(ROOT, "include", "ffnq.h")], flags))
    if not os.path.exists(exe):
        r = subprocess.run([HIPCC] + flags + ["-I", os.path.join(ROOT, "include")] + src + ["-o", exe + ".tmp"],
                           capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stderr[-3000:]
        os.replace(exe + ".tmp", exe)
    assert "ok" in run(exe)
