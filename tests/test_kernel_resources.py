"""Kernel resource records (no GPU needed): after TensorFold PR #1620's kernel records and its
merge discussion, where a register budget cured spill stores on the paged twins.

* No kernel of the build spills: zero scratch bytes per lane and no VGPR or SGPR spill, from the
  compiler's kernel-resource-usage remarks of the last build.
* The committed record profiles/kernel_resources.json matches the build: a kernel whose
  registers, LDS or occupancy change fails here until the record is rewritten
  (python -m paged_kv_cache_rows_amd.build --record).
"""
import json
import os

import pytest

from paged_kv_cache_rows_amd import build

REPORT = os.path.join(build.BUILD, "resource_usage.txt")


@pytest.fixture(scope="module")
def resources():
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES] + [os.path.join(build.ROOT, "include", "kvpaged.h")]
    if not os.path.exists(REPORT) or os.path.getmtime(REPORT) < max(os.path.getmtime(p) for p in srcs):
        build.build()
    return build.parse_resources(REPORT)


def test_every_kernel_is_reported(resources):
    names = " ".join(resources)
    for k in ("part_valu_kernel", "part_mfma_kernel", "merge_kernel", "rows_put_kernel", "pages_copy_kernel"):
        assert k in names
    for r in resources.values():
        assert set(r) == set(build.RESOURCE_FIELDS.values())


def test_no_kernel_spills(resources):
    bad = {n: r for n, r in resources.items() if r["scratch_bytes"] or r["vgpr_spill"] or r["sgpr_spill"]}
    assert not bad, f"kernels with scratch or spills: {bad}"


def test_the_committed_record_matches_the_build(resources):
    with open(build.RECORD_JSON) as f:
        record = json.load(f)
    assert set(record) == set(resources), "kernels added or removed: rewrite the record"
    diff = {n: (record[n], resources[n]) for n in resources if record[n] != resources[n]}
    assert not diff, f"kernel resources changed (rewrite the record): {diff}"
