"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/ are built with the host compilers (gcc, g++)
and run:
  - oracle_driver.c + oracle/oracle.c: every oracle function on small ragged
    inputs in exact-size buffers, with property checks;
  - abi_driver.cpp + the C ABI source (ck_api.cpp) + stub_launch.cpp: every
    entry point's validation, kernel dispatch and workspace carving, with host
    stand-ins for the kernel launchers that touch each row the real kernel
    would touch.
A third tiny program (a heap overflow, a signed overflow) checks that the
sanitizer runtimes are really active, so that a clean run means something.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined,float-cast-overflow",
         "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(not (shutil.which("gcc") and shutil.which("g++")),
                                reason="host compilers gcc/g++ not found")


def _build(tmp_path, name, compiler, std, sources, extra=(), flags=FLAGS):
    exe = str(tmp_path / name)
    cmd = [compiler, std, *flags, *extra, *sources, "-o", exe]
    if compiler == "gcc":
        cmd.append("-lm")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, f"build of {name} failed:\n{r.stderr}"
    return exe


def _run(exe, *args):
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=ENV)


def test_sanitizer_runtimes_are_active(tmp_path):
    """A one-byte heap overflow (AddressSanitizer alone) and a signed overflow
    (the undefined-behaviour set) are both reported: a clean driver run means
    these checks ran."""
    src = tmp_path / "bad.c"
    src.write_text("#include <limits.h>\n#include <stdlib.h>\n"
                   "int main(int argc, char **argv) {\n"
                   "  (void)argv;\n"
                   "  if (argc == 2) { volatile int i = INT_MAX; i = i + argc; return i == 0; }\n"
                   "  volatile char *p = malloc(16); p[15 + argc] = 1; free((void *)p); return 0; }\n")
    asan = _build(tmp_path, "bad_asan", "gcc", "-std=c11", [str(src)],
                  flags=["-O1", "-g", "-fsanitize=address", "-fno-sanitize-recover=all"])
    r = _run(asan)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr
    ub = _build(tmp_path, "bad_ub", "gcc", "-std=c11", [str(src)])
    r = _run(ub, "x")
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "oracle_driver", "gcc", "-std=c11",
                 [os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")],
                 extra=["-ffp-contract=off"])
    r = _run(exe)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr


def test_c_abi_under_asan_ubsan(tmp_path):
    exe = _build(tmp_path, "abi_driver", "g++", "-std=c++17",
                 [os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "stub_launch.cpp"),
                  os.path.join(ROOT, "packed_int4_convrot_amd", "csrc", "ck_api.cpp")],
                 extra=["-I" + os.path.join(ROOT, "include")])
    r = _run(exe)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr
