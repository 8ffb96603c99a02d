"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two builds made here, each run in its own process with its sanitizer runtime
preloaded (the interpreter itself is not instrumented):

- libh3attn.so with the host side of every source instrumented (the device
  code is unchanged; sanitizers are a host-only option of the HIP compiler),
  running the C-ABI tests: argument checks, workspace plans, RoPE table fill,
  error strings and the injected launch failure;
- the fp64 oracle (gcc), running its pins.

Any report (out-of-bounds access, use after free, signed overflow, misaligned
access, ...) aborts the child process and fails the test.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from audio_diffusion_transformer_amd import build as hbuild  # noqa: E402

SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_pytest(test_file, env_extra, preload):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", test_file)], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:] + r.stderr[-4000:])
    assert " passed" in r.stdout
    return r


def _exports(lib, prefix):
    r = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True)
    return [ln for ln in r.stdout.splitlines() if prefix in ln]


def test_abi_host_code_under_asan_ubsan(tmp_path):
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no clang AddressSanitizer runtime in this image")
    lib = str(tmp_path / "libh3attn_asan.so")
    hbuild.build(out=lib, extra=["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                 "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                                 "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan"])
    assert _exports(lib, "__asan_report"), "the host code is not instrumented"
    _run_pytest("test_abi_cpu.py", {"H3ATTN_LIB": lib}, rt[-1])


def test_oracle_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no gcc AddressSanitizer runtime in this image")
    lib = str(tmp_path / "liboracle_asan.so")
    src = os.path.join(ROOT, "oracle", "h3_oracle.c")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared", "-Wall",
                           "-Wno-unused-function", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", src, "-o", lib,
                           "-lm", "-lpthread"])
    assert _exports(lib, "__asan_report"), "the oracle is not instrumented"
    _run_pytest("test_oracle_pins.py", {"H3_ORACLE_LIB": lib}, asan)
