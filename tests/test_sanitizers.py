"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host-side C++
(CPU only, g++): the library's argument checks, workspace layouts and
admission queue (against a stub of the kernel launches), and the CPU oracle
with the seeded input generator.  Each driver under tests/sanitize/ exercises
every entry point with valid, degenerate and rejected arguments; a sanitizer
report aborts it.  Two planted errors check that the sanitizers are live.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "diffusion_drafter_verification_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")

FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-pthread"]
ENV = {"ASAN_OPTIONS": "detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _build(out: str, sources: list, extra: list = ()) -> None:
    cmd = ["g++"] + FLAGS + list(extra) + ["-o", out] + sources
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]


def _run(exe: str):
    env = dict(os.environ)
    env.update(ENV)
    return subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)


def test_host_code_is_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host")
    _build(exe, [os.path.join(SAN, "host_driver.cpp"), os.path.join(SAN, "launch_stub.cpp"),
                 os.path.join(CSRC, "adaflash_api.cpp"), os.path.join(CSRC, "adaflash_layout.cpp"),
                 os.path.join(CSRC, "adaflash_admission.cpp")],
           ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"])
    res = _run(exe)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-6000:]
    assert "host driver: 0 failed checks" in res.stdout


def test_oracle_and_generator_are_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle")
    _build(exe, [os.path.join(SAN, "oracle_driver.cpp"), os.path.join(ROOT, "oracle", "oracle.cpp"),
                 os.path.join(ROOT, "workloads", "gen.cpp")], ["-ffp-contract=off"])
    res = _run(exe)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-6000:]
    assert "oracle driver: 0 failed checks" in res.stdout


@pytest.mark.parametrize("body,report", [
    ("int* a = new int[4]; int i = argc + 3; a[i] = 1; int r = a[0]; delete[] a; return r;",
     ("heap-buffer-overflow", "insufficient space")),
    ("int x = 2147483647 - 1 + argc; x += 1; return x == 0;", ("signed integer overflow",)),
])
def test_sanitizers_catch_planted_errors(tmp_path, body, report):
    src = tmp_path / "planted.cpp"
    src.write_text("int main(int argc, char**) { " + body + " }\n")
    exe = str(tmp_path / "planted")
    _build(exe, [str(src)])
    res = _run(exe)
    assert res.returncode != 0
    assert any(r in res.stderr for r in report), res.stderr[-2000:]
