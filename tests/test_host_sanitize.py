"""The C-ABI layer (mla_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

mla_api.cpp is compiled with g++ and the sanitizers, linked with stand-ins for the kernel
launchers and the two HIP runtime queries it makes (tests/host_sanitize/stubs.cpp), and driven in a
child process that preloads the sanitizer runtime (tests/host_sanitize/driver.py): every entry
point is called with exactly sized host buffers, and the stand-ins read both ends of every range a
kernel would touch.  A wrong workspace carve-up, an output offset past its buffer, a signed overflow
in the size arithmetic or any other undefined behaviour ends the child with a sanitizer report.
Also checked: the same build reports a planted overrun (so the harness can fail at all).
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "deepseek_mla_latent_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                                reason="needs g++ and the HIP headers")


def _compile(out, sources, extra=()):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SAN, *extra, "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources, "-o", out,
           "-Wl,-z,defs"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(lib, *args):
    runtime = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    return subprocess.run([sys.executable, os.path.join(HERE, "driver.py"), lib, *args], capture_output=True,
                          text=True, env=env, timeout=300)


@pytest.fixture(scope="module")
def san_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("host_sanitize")
    return _compile(str(d / "libmla_api_san.so"), [os.path.join(CSRC, "mla_api.cpp"), os.path.join(HERE, "stubs.cpp")])


def test_c_abi_layer_is_clean_under_asan_and_ubsan(san_lib):
    r = _run(san_lib)
    assert r.returncode == 0 and "DRIVER OK" in r.stdout, (r.stdout[-3000:], r.stderr[-6000:])


def test_the_harness_reports_an_overrun(tmp_path):
    """A launcher stand-in that reads one element past the workspace must end the child with the
    AddressSanitizer report."""
    src = tmp_path / "stubs_overrun.cpp"
    text = open(os.path.join(HERE, "stubs.cpp")).read()
    # the range plan ends the workspace of the separate merge; 16 bytes past it is past any padding
    planted = text.replace("touch(row_plan, 16 + (size_t)rows * 8);\n  touch(o_lat",
                           "touch(row_plan, 16 + (size_t)rows * 8 + 16);\n  touch(o_lat", 1)
    assert planted != text
    src.write_text(planted.replace('#include "../../deepseek_mla_latent_amd/csrc/kernels.h"',
                                   f'#include "{os.path.join(CSRC, "kernels.h")}"'))
    lib = _compile(str(tmp_path / "libmla_api_overrun.so"), [os.path.join(CSRC, "mla_api.cpp"), str(src)])
    r = _run(lib)
    assert r.returncode == 86, (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
    assert "heap-buffer-overflow" in r.stderr
