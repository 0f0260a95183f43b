"""The host library under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

After colibri PR #1784, whose host code was run under ASan+UBSan: the C-ABI library's host code
(csrc/api.cpp: pool, lease queue, holder counts, shares, contiguous placement, argument checks)
is compiled with both sanitizers by g++, linked with the same gfx950 kernel objects as the
product build, and the host-side ABI tests (tests/test_abi_cpu.py) run against it with the
sanitizer runtimes preloaded into the interpreter; any report aborts the run.  A planted
overflow in a separate file proves the harness goes red.
"""
import os
import shutil
import subprocess
import sys

import pytest

from paged_kv_cache_rows_amd import build

ROOT = build.ROOT
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]
OPTS = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _runtime(name):
    p = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not _runtime("libasan.so") or not _runtime("libubsan.so"),
                                reason="g++ with the ASan/UBSan runtimes is needed")


def _env(lib):
    env = dict(os.environ, **OPTS)
    env["KVPAGED_LIB"] = lib
    env["LD_PRELOAD"] = ":".join([_runtime("libasan.so"), _runtime("libubsan.so")])
    return env


def test_abi_tests_pass_with_the_host_code_under_asan_and_ubsan(tmp_path):
    objs = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    api_o = str(tmp_path / "api.o")
    lib = str(tmp_path / "libkvpaged.so")
    cc = subprocess.run(["g++", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", "-c",
                         os.path.join(build.CSRC, "api.cpp"), "-o", api_o], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    ln = subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib, api_o, *objs,
                         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert ln.returncode == 0, ln.stderr
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the library is not instrumented"
    # every host-side ABI test except the one that removes the library altogether
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-k", "not without_the_library"],
                       cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]


def test_the_harness_catches_a_planted_overflow(tmp_path):
    src = tmp_path / "planted.cpp"
    src.write_text("#include <vector>\n#include <cstdio>\n"
                   "int main(int argc, char**) { std::vector<int> v(4, 1); volatile int i = 3 + argc;\n"
                   "  std::printf(\"%d\\n\", v.data()[i]); return 0; }\n")
    exe = str(tmp_path / "planted")
    cc = subprocess.run(["g++", *FLAGS, str(src), "-o", exe], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    r = subprocess.run([exe], env=dict(os.environ, **OPTS), capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
