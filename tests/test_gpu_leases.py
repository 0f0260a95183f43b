"""GPU tests of the contiguous lease policy (TensorFold PR #1620, first review, which suggests
keeping the full layers in one unbroken run of pages while the pool has space to spare).

Streams that grow side by side, a page at a time, lease under KV_LEASE_CONTIGUOUS from a pool
that ends up nearly full, so most tables are one run of adjacent ids and some spill into a
second run.  The policy moves pages, never results: decode and verify through these tables
are byte-equal to the same caches built on shuffled pages, and match the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_support import assert_close, attend, oracle_for, remember, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _runs(row):
    return 1 + int((np.diff(row) != 1).sum())


def _w(P):
    return workloads.Workload(name="contig", streams=5, kv_heads=2, group=8, head_dim=128, page_size=P, rows=1,
                              lengths=[2900, 1800, 3300, 700, 2500], spare_frac=0.05, min_spares=1, seed=71)


@pytest.mark.parametrize("P", [64, 37])
def test_contiguous_leases_give_the_same_bytes_as_shuffled_pages(P):
    w = _w(P)
    say(f"contiguous leases P={P}: lengths {w.lengths}, pool {w.pool_pages}")
    ks, vs = workloads.kv_history(w)
    caches = []
    for kind in ("contiguous", "shuffled"):
        if kind == "contiguous":
            c = staging.make_cache(w, order=workloads.identity_order(w.pool_pages),
                                   lease_policy=binding.KV_LEASE_CONTIGUOUS, grow_in_turn=1)
        else:
            c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 7101))
        staging.write_history(c, ks, vs)
        caches.append(remember(c, ks, vs))
    runs = [_runs(caches[0].table_host[s][:w.pages_for(L)]) for s, L in enumerate(w.lengths)]
    say(f"runs per stream: {runs}")
    assert min(runs) == 1 and max(runs) >= 2          # contiguous where it fits, spilled where not
    for mode, rows in (("decode", 1), ("verify", 4)):
        q = workloads.queries(w, rows=rows, salt=rows).cuda()
        a = attend(mode, caches[0], q)
        b = attend(mode, caches[1], q)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{mode}: contiguous != shuffled bytes"
        assert_close(a, oracle_for(caches[0], q), f"{mode} P={P} contiguous leases")
