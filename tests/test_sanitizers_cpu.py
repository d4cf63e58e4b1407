"""Host-side sanitizer runs (no GPU): AddressSanitizer and UndefinedBehaviorSanitizer
on the CPU code of this repository.

* The oracle, built with gcc -fsanitize=address,undefined, runs its whole pin suite.
* The library's host code (argument validation, workspace sizing, dispatch; the device
  code is unchanged), built with host-only sanitizers, runs the ABI and binding tests.
* A planted out-of-bounds write in a copy of the oracle must be reported, which shows
  the sanitizer is really active in these runs.

Each run is a child process with the sanitizer runtime preloaded (ahead of anything the
environment already preloads) and leak detection off (the interpreter's own allocations
are not ours); any report is written to a log file and fails the test."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "bitlinear_oracle.c")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _runtime(compiler, name):
    r = subprocess.run([compiler, "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _run_sanitized(runtime, args, env_extra, logdir):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:log_path=" + os.path.join(logdir, "asan")
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:log_path=" + os.path.join(logdir, "ubsan")
    env.update(env_extra)
    # -s: the sanitizers' reports go to the child's own stderr, which is kept here (a
    # report ends the process, so pytest's capture of it would be lost)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                        *args], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = "".join(line + "\n" for line in r.stderr.splitlines()
                      if "runtime error" in line or "AddressSanitizer" in line)
    for f in sorted(glob.glob(os.path.join(logdir, "asan*")) + glob.glob(os.path.join(logdir, "ubsan*"))):
        reports += open(f).read()
    return r, reports


def _build_oracle(src_text, out_dir):
    c = os.path.join(out_dir, "oracle.c")
    so = os.path.join(out_dir, "oracle_san.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-w", "-o", so, c, "-lm"], check=True)
    return so


@pytest.fixture(scope="module")
def gcc_asan():
    rt = _runtime("gcc", "libasan.so")
    if rt is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return rt


def test_oracle_pins_under_asan_and_ubsan(gcc_asan):
    with tempfile.TemporaryDirectory() as d:
        so = _build_oracle(open(ORACLE_SRC).read(), d)
        r, reports = _run_sanitized(gcc_asan, [os.path.join(ROOT, "tests", "test_oracle.py")],
                                    {"ORACLE_LIB": so}, d)
    assert r.returncode == 0 and not reports, r.stdout[-3000:] + r.stderr[-3000:] + reports


def test_sanitizer_reports_a_planted_overflow(gcc_asan):
    # the exact sum's limb loop one past its 18-word accumulator (a stack array)
    src = open(ORACLE_SRC).read()
    old = "for (int i = li; i < SQ_LIMBS; ++i) {"
    assert old in src
    with tempfile.TemporaryDirectory() as d:
        so = _build_oracle(src.replace(old, "for (int i = li; i <= SQ_LIMBS; ++i) {"), d)
        r, reports = _run_sanitized(
            gcc_asan, [os.path.join(ROOT, "tests", "test_oracle.py"), "-k", "sum_of_squares_hand"],
            {"ORACLE_LIB": so}, d)
    assert r.returncode != 0 and reports, r.stdout[-2000:] + r.stderr[-2000:]


def test_library_host_code_under_asan_and_ubsan():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    rt = _runtime(HIPCC, "libclang_rt.asan-x86_64.so")
    if rt is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    from ternary_weight_quantized_bitlinear_amd import build
    flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as d:
        lib = build.build(out=os.path.join(d, "libbitlinear_san.so"), build_dir=os.path.join(d, "o"),
                          extra=flags)
        r, reports = _run_sanitized(rt, [os.path.join(ROOT, "tests", "test_abi_cpu.py"),
                                         os.path.join(ROOT, "tests", "test_binding_cpu.py")],
                                    {"BITLINEAR_LIB": lib}, d)
    assert r.returncode == 0 and not reports, r.stdout[-3000:] + r.stderr[-3000:] + reports
