"""GPU parity tests at large sizes: one stream of 262,144 keys (decode on the VALU path and a
4-row verify on the MFMA path, with hundreds of splits), and a stream whose pages all have ids
above 65,536 in a pool of 70,000 pages, so that page offsets need more than 32 bits of
elements.  Every output is compared in full with the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_support import assert_close, attend, oracle_for, say
from paged_kv_cache_rows_amd import staging, workloads

pytestmark = pytest.mark.gpu

LONG = 262144


def _long(P, rows):
    return workloads.Workload(name="long", streams=1, kv_heads=1, group=8, head_dim=128, page_size=P, rows=rows,
                              lengths=[LONG], spare_frac=0.02, min_spares=2, seed=91)


@pytest.mark.parametrize("P", [64, 37])
def test_decode_over_262144_keys(P):
    w = _long(P, 1)
    say(f"decode over {LONG} keys, pages of {P}, pool {w.pool_pages}")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 9101))
    ks, vs = workloads.kv_history(w)
    staging.write_history(c, ks, vs)
    q = workloads.queries(w).cuda()
    out = attend("decode", c, q)
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q), f"decode L={LONG} P={P}")


def test_verify_over_262144_keys():
    w = _long(64, 4)
    say(f"verify (4 rows, MFMA) over {LONG} keys")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 9102))
    ks, vs = workloads.kv_history(w)
    staging.write_history(c, ks, vs)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q)
    assert_close(out, oracle_for(c, q), f"verify R=4 L={LONG}")


def test_pages_with_ids_above_65536():
    # 1,250 pages of 16 at the top of a 70,000-page pool: page p starts p * 2048 elements in
    w = workloads.Workload(name="high_ids", streams=1, kv_heads=1, group=8, head_dim=128, page_size=16, rows=1,
                           lengths=[20000], spare_frac=55.0, min_spares=2, seed=92)
    assert w.pool_pages == 70000
    order = np.arange(w.pool_pages, dtype=np.int32)[::-1].copy()
    say(f"pages with high ids: pool {w.pool_pages}")
    c = staging.make_cache(w, order=order)
    assert c.table_host[0][:w.pages_for(20000)].min() > 65536
    ks, vs = workloads.kv_history(w)
    staging.write_history(c, ks, vs)
    for rows, mode in ((1, "decode"), (4, "verify")):
        q = workloads.queries(w, rows=rows, salt=rows).cuda()
        out = attend(mode, c, q)
        assert_close(out, oracle_for(c, q), f"{mode} on pages above 65536")
