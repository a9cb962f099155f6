"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle is built with g++ -fsanitize=address,undefined and the pin suite
runs against it; libvs.so is built with its host code sanitised (hipcc
-Xarch_host -fsanitize=...) and the ABI checks (argument validation,
workspace sizes, the exported symbols) run against it. Each suite runs in a
subprocess with the matching runtime preloaded and every report fatal, so an
out-of-bounds access, a use after free, a signed overflow or an invalid enum
load in host code fails the test with the sanitizer's report.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG_ASAN = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
SAN_OPTIONS = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run(args, env_extra, timeout):
    env = dict(os.environ, **SAN_OPTIONS, **env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc's sanitizer runtimes are not installed")
    lib = oracle.build(force=True, path=str(tmp_path / "liboracle.so"), sanitize=True)
    out = _run(["tests/test_oracle_pins.py", "-k", "not exhaustive"],
               {"DTS_ORACLE_LIB": lib, "LD_PRELOAD": f"{asan} {ubsan}"}, timeout=600)
    assert " passed" in out


def test_abi_under_asan_ubsan(tmp_path):
    if not os.path.exists(CLANG_ASAN):
        pytest.skip("clang's ASan runtime is not installed")
    from decode_token_sampling_amd import build
    lib = build.build_host_sanitized(str(tmp_path))
    out = _run(["tests/test_abi_cpu.py"], {"VS_LIBRARY": lib, "LD_PRELOAD": CLANG_ASAN},
               timeout=300)
    assert " passed" in out
