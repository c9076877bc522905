"""Host-code sanitizer runs (CPU only, no GPU call).

- The C oracle built by gcc with AddressSanitizer and UndefinedBehaviorSanitizer
  (recovery off) runs the oracle's pins (tests/test_oracle_pins.py,
  tests/test_quant_oracle.py).
- The HIP library built from the same sources with both sanitizers on hipcc's
  host pass only (argument checks, launch planning, scratch layout; the device
  code is compiled as usual) runs the C-ABI host-check tests
  (tests/test_abi_cpu.py).

Each run is a subprocess with the matching sanitizer runtime preloaded into the
Python interpreter; a non-zero exit or any sanitizer report fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp4_mqa_scoring_amd", "csrc")
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "SUMMARY: UndefinedBehaviorSanitizer")


def _runtime(compiler, name):
    out = subprocess.run([compiler, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def _run_tests(tests, env_extra, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = ":".join(preload)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"      # the interpreter itself keeps memory at exit
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests], cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=900)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    for rep in REPORTS:
        assert rep not in text, text[-4000:]
    assert " passed" in text, text[-2000:]


def _instrumented(path):
    syms = subprocess.run(["nm", "-D", path], capture_output=True, text=True).stdout
    return "__asan_" in syms and "__ubsan_" in syms


def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    asan, ubsan = _runtime(gcc, "libasan.so"), _runtime(gcc, "libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not found")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                    os.path.join(ROOT, "oracle", "oracle.c"), "-o", lib, "-lm"], check=True)
    assert _instrumented(lib)
    _run_tests(["tests/test_oracle_pins.py", "tests/test_quant_oracle.py"], {"MQA_ORACLE_LIB": lib},
               [asan, ubsan])


def test_library_host_checks_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from fp4_mqa_scoring_amd import build as b
    try:
        hipcc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    rt = _runtime(os.path.join(os.path.dirname(hipcc), "hipcc"), "libclang_rt.asan-x86_64.so")
    if rt is None:
        pytest.skip("clang sanitizer runtime not found")
    lib = str(tmp_path / "libmqa_fp4_san.so")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in b.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + host_san
    subprocess.run([hipcc, *flags, "-I", os.path.join(ROOT, "include"), *b.SOURCES, "-o", lib], check=True,
                   capture_output=True)
    assert _instrumented(lib)
    _run_tests(["tests/test_abi_cpu.py"], {"MQA_ABI_TEST_LIB": lib}, [rt])
