"""Host check of the kernels' key ranges, page lookups and merge spans (no GPU needed).

tests/key_ranges_check.cpp is linked with the library's own host objects (its launch plan) and
uses the range, lookup-mode and merge-span functions the kernels call.  It walks the load steps
of every workgroup for about 900 call shapes and 22,000 device lengths, among them lengths
above max_seq_len (caller errors, which the kernels read as max_seq_len) and full layers of
exactly as many pages as the kernels cache; at the longest stream and widest window a call may
describe (KV_MAX_SEQ_LEN) it checks the ranges and merge spans of every workgroup.  It is built
with the signed-overflow check of UndefinedBehaviorSanitizer, so a 32-bit overflow in those
functions stops it.  Three planted mistakes must be reported.
"""
import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_rows_amd import build

ROOT = build.ROOT
SRC = os.path.join(ROOT, "tests", "key_ranges_check.cpp")
OBJS = ["api.o", "kernels_valu.o", "kernels_mfma.o", "kernels_io.o", "scratch.o"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                                reason="g++ and the ROCm headers are needed")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    objs = [os.path.join(build.BUILD, o) for o in OBJS]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    exe = str(tmp_path_factory.mktemp("ranges") / "key_ranges_check")
    cc = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-fsanitize=signed-integer-overflow",
                         "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                         f"-I{build.CSRC}", SRC, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                         "-Wl,-rpath,/opt/rocm/lib", "-o", exe], capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr[-4000:]
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=300)
    m = re.search(r"shapes (\d+) lengths (\d+) workgroups (\d+) rows (\d+) absent-entry rows (\d+) "
                  r"outside-cache lookups (\d+) violations (\d+)", r.stdout)
    assert m, r.stdout[-2000:] + r.stderr[-2000:]
    return r, [int(x) for x in m.groups()]


def test_every_workgroup_reads_its_own_pages_and_the_pieces_tile_the_keys(checker):
    r, (shapes, lengths, wgs, rows, absent, outside, bad) = _run(checker)
    assert bad == 0 and r.returncode == 0, r.stdout[-3000:]
    assert shapes > 1000 and lengths > 20000 and wgs > 10**7 and rows > 10**8
    # the last load step of a full layer of exactly the cached number of pages (pages of 37 or
    # 100 keys) looks up entries past the cache: those rows must read an absent page, not LDS
    # beyond the table
    assert outside > 0 and absent >= outside


@pytest.mark.parametrize("plant, message", [("merge", "merge does not hold each key of its row once"),
                                            ("cache", "used key read through an absent entry"),
                                            ("put", "a new row is not written exactly once")])
def test_planted_mistakes_are_reported(checker, plant, message):
    r, (*_, bad) = _run(checker, "--plant", plant)
    assert r.returncode == 1 and bad > 0 and message in r.stdout, r.stdout[-2000:]


def test_an_overflow_in_the_range_functions_stops_the_checker(checker):
    r = subprocess.run([checker, "--plant", "overflow"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "signed integer overflow" in r.stderr and "internal.h" in r.stderr, \
        (r.returncode, r.stderr[-2000:])
