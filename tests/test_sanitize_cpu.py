"""The host half of libtpshard (argument validation, shard splits,
accounting, options) under AddressSanitizer and UndefinedBehaviorSanitizer,
driven on the CPU by tests/sanitize/abi_driver.c: every call is host-only or
rejected before any launch, so no GPU is needed.  The device code is built
as usual (the sanitizers apply to the host compilation only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "attention_column_gemm_amd", "csrc", "tp_shard.hip")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "abi_driver.c")
INC = os.path.join(ROOT, "include")


@pytest.mark.slow
def test_host_validation_under_asan_and_ubsan(tmp_path):
    from attention_column_gemm_amd.build import HIPCC_FLAGS, hipcc
    cc = shutil.which("clang") or "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(cc):
        pytest.skip("clang is not available")
    lib = tmp_path / "libtpshard_san.so"
    flags = [f for f in HIPCC_FLAGS if f not in ("-O3",)]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    r = subprocess.run([hipcc(), *flags, "-O1", "-g", *san, SRC, "-o", str(lib)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = tmp_path / "abi_driver"
    r = subprocess.run([cc, "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-I", INC, DRIVER, str(lib), f"-Wl,-rpath,{tmp_path}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all expectations hold" in r.stdout
