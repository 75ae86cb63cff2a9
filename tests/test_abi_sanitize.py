"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU, no GPU needed).

Every library source is compiled with the sanitizers on its host half only
(the device half is built unoptimized: it is never launched here) and linked
with ``abi_sanitize_driver.c``, which calls every entry point with arguments its
validation must refuse -- NULL pointers, ragged or negative sizes, and sizes at
the ends of int64_t, where the validation's own products and sums would
overflow -- and checks each documented status code.  Signed overflow, an
out-of-bounds access or a leak in the host code aborts the driver."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_sanitize_driver.c")


def _toolchain():
    from moe_token_block_amd import build as b
    try:
        cc = b.hipcc()
    except RuntimeError:
        return None
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(cc)))
    for cxx in (os.path.join(rocm, "llvm", "bin", "clang++"), "/opt/rocm/llvm/bin/clang++"):
        if os.path.exists(cxx):
            return b, cc, cxx, rocm
    return None


def test_abi_validation_under_sanitizers(tmp_path):
    tc = _toolchain()
    if tc is None:
        pytest.skip("hipcc or ROCm's clang++ not found")
    b, cc, cxx, rocm = tc
    host_sanitizers = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = ["-O0", "-Xarch_host", "-O1", "-g", "-std=c++17", f"--offload-arch={b.ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"] + host_sanitizers
    procs, objs = [], []
    for src in b.SOURCES:
        obj = str(tmp_path / src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [cc] + flags + ["-c", os.path.join(b.CSRC, src), "-o", obj]
        procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate(timeout=600)
        assert p.returncode == 0, out[-4000:]

    exe = str(tmp_path / "abi_sanitize_driver")
    link = [cxx, "-x", "c", DRIVER, "-x", "none", "-g", "-fsanitize=address,undefined",
            "-fno-sanitize-recover=all"] + objs
    link += ["-L" + os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"),
             "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr

    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr
    shutil.rmtree(tmp_path, ignore_errors=True)
