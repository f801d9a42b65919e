"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code, on the CPU.

Two programs are built with gcc/g++ and run here:
  - the C oracle (oracle/gdn_oracle.c) under a driver that runs the forward and
    the decode step, real and complex, over ragged lengths with and without an
    initial state (tests/sanitize/oracle_driver.c);
  - the C-ABI layer (gdn_api.cpp, rebuilt with the sanitizers) linked with the
    kernel objects of the last build, under a driver that sends every entry
    point arguments that fail validation, plus the calls that have nothing to
    do (tests/sanitize/abi_driver.cpp).  No call reaches a kernel, so no GPU is
    needed; the HIP runtime is linked but never asked to launch.
Any sanitizer report ends the program with a non-zero status.  The last tests
plant a heap overflow and a signed overflow in throw-away programs to show
that each sanitizer is live.  Device code is not instrumented (GPU sanitizers are not
available for it); only host code is.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
ROCM = "/opt/rocm"

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nstatus {r.returncode}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    _run(["gcc", "-std=c99", "-fopenmp"] + SAN +
         [os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=ENV)
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr


def _kernel_objects():
    from linear_attention_sequence_gated_amd import build as gbuild
    objs = [os.path.join(gbuild.OBJDIR, os.path.splitext(s)[0] + ".o") for s in gbuild.SOURCES if s != "gdn_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        gbuild.build()
    return objs


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")), reason="HIP runtime not found")
def test_abi_layer_under_asan_ubsan(tmp_path):
    objs = _kernel_objects()
    api = str(tmp_path / "gdn_api.o")
    drv = str(tmp_path / "abi_driver.o")
    exe = str(tmp_path / "abi_asan")
    inc = ["-I", os.path.join(ROOT, "include")]
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")] + inc + SAN +
         ["-c", os.path.join(ROOT, "linear_attention_sequence_gated_amd", "csrc", "gdn_api.cpp"), "-o", api])
    _run(["g++", "-std=c++17"] + inc + SAN + ["-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                                               "-o", drv])
    _run(["g++"] + SAN + [drv, api] + objs +
         ["-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    r = _run([exe], env=ENV)
    assert "all checks passed" in r.stdout


@pytest.mark.parametrize("flag,body,report", [
    ("-fsanitize=address", "volatile int *p = malloc(4 * sizeof(int)); p[argc + 3] = 1; free((void *)p);",
     "heap-buffer-overflow"),
    ("-fsanitize=undefined", "volatile int x = INT_MAX; x = x + argc;", "signed integer overflow"),
])
def test_sanitizer_build_is_live(tmp_path, flag, body, report):
    """A planted heap overflow and a planted signed overflow must each be reported, or the tests above prove
    nothing."""
    src = tmp_path / "planted.c"
    src.write_text("#include <limits.h>\n#include <stdlib.h>\nint main(int argc, char **argv) {(void)argv; "
                   + body + " return 0;}\n")
    exe = str(tmp_path / "planted")
    _run(["gcc", flag, "-fno-sanitize-recover=all", "-g", "-O1", str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode != 0
    assert report in r.stderr
