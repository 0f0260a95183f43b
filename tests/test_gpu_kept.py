"""GPU tests of kept states and page reuse (TensorFold PR #1620, opening description, Kept
states bullet; the model test's "a kept state's resume and reused pages").

* kv_pages_copy is byte-equal to the oracle's page copy.
* A stream's state kept by copying its pages onto freshly leased ones reads back the same cache:
  attention through the kept table equals attention through the original at that length, byte
  for byte, after the original has moved on; and both match the oracle.
* Released pages handed to another stream still hold the old stream's rows; attention over the
  new stream never reads them (stale, finite data in unused slots must not leak either).
* A prefix shared between two streams (kv_page_share) serves both, and outlives its first
  holder: its pages are not handed out again while the second still holds them.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import assert_close, expected_pool, new_cache, oracle_from_history, pool_bits, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="kept", streams=3, kv_heads=2, group=4, head_dim=128, page_size=64, rows=1,
                lengths=[900, 300, 900], spare_frac=0.3, min_spares=4, seed=51)
    base.update(kw)
    return workloads.Workload(**base)


@pytest.mark.parametrize("P,D", [(64, 128), (37, 512), (512, 128)])
def test_pages_copy_bytes_equal_the_oracle_copy(P, D):
    w = _w(page_size=P, head_dim=D, lengths=[2 * P + 5, P, 3 * P])
    c, _, _ = new_cache(w)
    kb, vb = expected_pool(c)                               # the oracle's scatter of the history
    gk, gv = pool_bits(c)
    assert np.array_equal(gk, kb) and np.array_equal(gv, vb)
    rng = np.random.default_rng(P + D)
    ids = rng.permutation(w.pool_pages)
    n = w.pool_pages // 2
    src, dst = ids[:n].astype(np.int32), ids[n:2 * n].astype(np.int32)
    src[0] = w.pool_pages + 3                               # out of the pool: skipped
    binding.pages_copy(c.pool, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    kg, vg = pool_bits(c)
    assert np.array_equal(kg, oracle.copy_pages(kb, src, dst))
    assert np.array_equal(vg, oracle.copy_pages(vb, src, dst))


def test_kept_state_resumes_byte_equal_after_the_original_moves_on():
    w = _w()
    ks, vs = workloads.kv_history(w)
    L0 = 600                                                # the state to keep: stream 0 at 600
    # stream 0's history so far is 600 rows (the leases cover 900)
    c0, _, _ = new_cache(w, history=False)
    staging.write_history(c0, ks, vs, upto=[L0, 300, 0])
    dev = c0.table.device
    kept_ids = c0.pool.lease(2, -(-L0 // w.page_size))     # stream 2's slot holds the kept state
    src = torch.tensor(c0.table_host[0][:len(kept_ids)], dtype=torch.int32, device=dev)
    dst = torch.tensor(kept_ids, dtype=torch.int32, device=dev)
    binding.pages_copy(c0.pool, src, dst)
    q = workloads.normal_bf16((1, 1, w.q_heads, w.head_dim), 61).to(dev)
    seq = torch.tensor([L0], dtype=torch.int32, device=dev)
    before = binding.decode(c0.pool, q, c0.table[0:1], seq, L0)
    # the original moves on: 200 more rows
    t0 = c0.table[0:1]
    kn = ks[0][L0:L0 + 200][None].contiguous().to(dev)
    vn = vs[0][L0:L0 + 200][None].contiguous().to(dev)
    binding.rows_put(c0.pool, t0, torch.tensor([L0 + 200], dtype=torch.int32, device=dev), kn, vn, L0 + 200)
    kept_table = torch.full((1, c0.table.shape[1]), -1, dtype=torch.int32, device=dev)
    kept_table[0, :len(kept_ids)] = dst
    resumed = binding.decode(c0.pool, q, kept_table, seq, L0)
    moved = binding.decode(c0.pool, q, t0, torch.tensor([L0 + 200], dtype=torch.int32, device=dev), L0 + 200)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), resumed.view(torch.int16))
    assert_close(resumed, oracle_from_history(ks[:1], vs[:1], q, [L0]), "kept state at 600")
    assert_close(moved, oracle_from_history(ks[:1], vs[:1], q, [L0 + 200]), "original at 800")


def test_released_pages_reused_by_another_stream_leak_nothing():
    # stream 0 fills its pages, releases them; stream 1 leases them and writes a shorter history,
    # so its last page still holds stream 0's (finite) rows past stream 1's length
    w = workloads.Workload(name="reuse", streams=2, kv_heads=2, group=4, head_dim=128, page_size=64, rows=1,
                           lengths=[640, 611], spare_frac=0.0, min_spares=0, seed=52)
    w2 = dataclass_replace(w, lengths=[640, 1])             # 10 + 1 pages, no spares
    c = staging.make_cache(w2, order=workloads.identity_order(w2.pool_pages), lengths=[640, 1])
    ks0, vs0 = workloads.kv_history(w2)
    staging.write_history(c, ks0, vs0, upto=[640, 0])
    released = c.pool.stream_pages(0)
    c.pool.release(0)
    c.pool.release(1)
    ids = c.pool.lease(1, 10)                                # every page; stream 0's come back too
    assert set(released) <= set(ids)
    dev = c.table.device
    table = torch.tensor([ids], dtype=torch.int32, device=dev)
    ks1, vs1 = workloads.kv_history(dataclass_replace(w, lengths=[611]), salt=5)
    for c0 in range(0, 611, 200):
        c1 = min(611, c0 + 200)
        binding.rows_put(c.pool, table, torch.tensor([c1], dtype=torch.int32, device=dev),
                         ks1[0][c0:c1][None].contiguous().to(dev), vs1[0][c0:c1][None].contiguous().to(dev), c1)
    q = workloads.normal_bf16((1, 4, w.q_heads, w.head_dim), 62).to(dev)
    seq = torch.tensor([611], dtype=torch.int32, device=dev)
    out = binding.verify(c.pool, q, table, seq, 611)
    torch.cuda.synchronize()
    kb, _ = pool_bits(c)
    last = ids[(611 - 1) // 64]
    assert not (kb[last, :, 611 % 64:] == workloads.NAN_BITS).all()     # stale rows really are there
    assert_close(out, oracle_from_history(ks1, vs1, q, [611]), "reused pages")


def test_shared_prefix_serves_both_streams_and_outlives_its_first_holder():
    # stream 0 writes 700 rows; stream 1 shares its 10 full pages (640 rows), gives the partly
    # filled 11th page its own copy, and continues from row 660 with rows of its own
    P = 64
    w = workloads.Workload(name="share", streams=3, kv_heads=2, group=4, head_dim=128, page_size=P, rows=1,
                           lengths=[700, 860, 1], spare_frac=0.0, min_spares=0, seed=53)
    ks, vs = workloads.kv_history(w)
    pool = binding.Pool(40, P, 2, 128, max_streams=3)
    dev = pool.k_pages.device

    def table_of(ids):
        t = torch.full((1, 16), -1, dtype=torch.int32, device=dev)
        t[0, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        return t

    def put(table, rows_k, rows_v, lo, hi):
        binding.rows_put(pool, table, torch.tensor([hi], dtype=torch.int32, device=dev),
                         rows_k[lo:hi][None].contiguous().to(dev), rows_v[lo:hi][None].contiguous().to(dev), hi)

    ids0 = pool.lease(0, 11)
    t0 = table_of(ids0)
    put(t0, ks[0], vs[0], 0, 700)
    pool.share(0, 1, 10)
    own = pool.lease(1, 4)
    binding.pages_copy(pool, torch.tensor([ids0[10]], dtype=torch.int32, device=dev),
                       torch.tensor([own[0]], dtype=torch.int32, device=dev))
    ids1 = pool.stream_pages(1)
    assert ids1 == ids0[:10] + own
    t1 = table_of(ids1)
    put(t1, ks[1], vs[1], 660, 860)
    hist_k = [ks[0][:700], torch.cat([ks[0][:660], ks[1][660:860]])]
    hist_v = [vs[0][:700], torch.cat([vs[0][:660], vs[1][660:860]])]
    q = workloads.normal_bf16((2, 1, w.q_heads, 128), 63).to(dev)
    out0 = binding.decode(pool, q[0:1].contiguous(), t0, torch.tensor([700], dtype=torch.int32, device=dev), 700)
    out1 = binding.decode(pool, q[1:2].contiguous(), t1, torch.tensor([860], dtype=torch.int32, device=dev), 860)
    torch.cuda.synchronize()
    ref = oracle_from_history(hist_k, hist_v, q, [700, 860])
    assert_close(out0, ref[0:1], "stream 0 through its own pages")
    assert_close(out1, ref[1:2], "stream 1 through the shared prefix")
    # the first holder leaves: only its unshared 11th page returns; another stream takes every
    # free page and overwrites it; stream 1 reads the same bytes as before
    pool.release(0)
    assert pool.free_count() == 40 - len(ids1)
    ids2 = pool.lease(2, pool.free_count())
    assert not set(ids2) & set(ids1)
    noise = workloads.normal_bf16((len(ids2), 2, P, 128), 64).to(dev)
    sel = torch.tensor(ids2, dtype=torch.long, device=dev)
    pool.k_pages[sel] = noise
    pool.v_pages[sel] = noise
    again = binding.decode(pool, q[1:2].contiguous(), t1, torch.tensor([860], dtype=torch.int32, device=dev), 860)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), again.view(torch.int16))
    pool.release(1)
    pool.release(2)
    assert pool.free_count() == 40


def dataclass_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)
