"""GPU tests at the edges of the kernels' page lookups and lengths, through the C ABI.

* Full layers whose table is exactly as long as the kernels' LDS cache of table entries (160
  pages), with pages of 37 or 100 keys: the last load step of a stream then reaches past its
  last page, and the rows there must come from an absent page (read, then masked out), never
  from LDS past the cached entries.  The outputs must match the oracle and the fused decode row
  write must reach page 159.
* Device lengths above max_seq_len, a caller error: every kernel reads such a length as
  max_seq_len, so the call gives exactly the result of the same call at max_seq_len, and a
  negative length gives the zeros of an empty stream.

The host-side walk of the same lookups over many more shapes is tests/test_key_ranges.py.
"""
import pytest
import torch

from gpu_support import (assert_close, oracle_for, oracle_from_history, pool_bits, poisoned_workspace, say,
                         new_cache)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu

CACHED_PAGES = 160
INT32_MAX = 2**31 - 1


def _w(D, G, R, P, lengths, seed=71):
    return workloads.Workload(name="bounds", streams=len(lengths), kv_heads=2 if D == 128 else 1, group=G,
                              head_dim=D, page_size=P, rows=R, lengths=lengths, spare_frac=0.2, min_spares=2,
                              seed=seed)


def _call(entry, c, q, seq, max_seq_len, **kw):
    fn = {"decode": binding.decode, "verify": binding.verify, "prefill": binding.prefill}[entry]
    out = fn(c.pool, q, c.table, seq, max_seq_len, workspace=poisoned_workspace(c, q.shape[1], q.shape[2]), **kw)
    torch.cuda.synchronize()
    return out


# (entry, D, G, R, P): VALU decode and verify (R G < 16), MFMA verify and prompt chunk
CASES = [("decode", 128, 8, 1, 37), ("decode", 128, 8, 1, 100), ("decode", 512, 12, 1, 37),
         ("decode", 512, 12, 1, 100), ("verify", 128, 4, 3, 37), ("verify", 128, 4, 3, 100),
         ("verify", 128, 8, 8, 37), ("verify", 128, 16, 4, 37), ("verify", 512, 8, 4, 37),
         ("prefill", 128, 8, 32, 37)]


@pytest.mark.parametrize("entry,D,G,R,P", CASES)
def test_full_layer_of_exactly_the_cached_pages(entry, D, G, R, P):
    full = CACHED_PAGES * P
    lengths = [full, full - 5, full - P - 1]
    w = _w(D, G, R, P, lengths)
    assert w.table_stride == CACHED_PAGES
    say(f"cached-pages layer: {entry} D={D} G={G} R={R} P={P} lengths {lengths}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = _call(entry, c, q, c.seq_len, c.max_seq_len)
    assert_close(out, oracle_for(c, q), f"{entry} D={D} G={G} R={R} P={P} at {CACHED_PAGES} pages")


@pytest.mark.parametrize("D,G,P", [(128, 8, 37), (512, 12, 100), (128, 16, 37)])
def test_decode_put_into_the_last_cached_page(D, G, P):
    full = CACHED_PAGES * P
    lengths = [full, full - 3]
    w = _w(D, G, 1, P, lengths, seed=72)
    say(f"decode_put at {CACHED_PAGES} pages: D={D} G={G} P={P}")
    ks, vs = workloads.kv_history(w)
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 7201))
    staging.write_history(c, ks, vs, upto=[L - 1 for L in lengths])
    dev = c.table.device
    k_new = torch.stack([ks[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    v_new = torch.stack([vs[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    q = workloads.queries(w).cuda()
    out = binding.decode_put(c.pool, q, c.table, c.seq_len, max(lengths), k_new, v_new,
                             workspace=poisoned_workspace(c, 1, w.q_heads))
    torch.cuda.synchronize()
    assert_close(out, oracle_from_history(ks, vs, q, lengths), f"decode_put D={D} G={G} P={P}")


@pytest.mark.parametrize("entry,D,G,R,P", [("decode", 128, 8, 1, 512), ("decode", 128, 8, 1, 37),
                                           ("decode", 512, 4, 1, 64), ("verify", 128, 4, 3, 64),
                                           ("verify", 128, 8, 8, 512), ("verify", 512, 8, 4, 37),
                                           ("prefill", 128, 8, 64, 64)])
def test_length_above_max_seq_len_reads_as_max_seq_len(entry, D, G, R, P):
    M = 3000
    w = _w(D, G, R, P, [M, M, M], seed=73)
    say(f"length above max_seq_len: {entry} D={D} G={G} R={R} P={P}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    dev = c.table.device
    ref = _call(entry, c, q, c.seq_len, M)
    assert_close(ref, oracle_for(c, q), f"{entry} at max_seq_len")
    over = torch.tensor([M + 9, INT32_MAX, -5], dtype=torch.int32, device=dev)
    got = _call(entry, c, q, over, M)
    assert torch.equal(got[:2].view(torch.int16), ref[:2].view(torch.int16)), "a length above max_seq_len"
    assert not got[2].float().abs().any(), "a negative length must give an empty stream's zeros"


def test_decode_put_with_a_length_above_max_seq_len_writes_position_max_seq_len_minus_1():
    M = 2000
    w = _w(128, 8, 1, 64, [M, M], seed=74)
    ks, vs = workloads.kv_history(w)
    order = workloads.free_order(w.pool_pages, 7401)
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=[M - 1, M - 1])
        caches.append(c)
    a, b = caches
    dev = a.table.device
    k_new = torch.stack([ks[s][M - 1:M] for s in range(2)]).to(dev).contiguous()
    v_new = torch.stack([vs[s][M - 1:M] for s in range(2)]).to(dev).contiguous()
    q = workloads.queries(w).cuda()
    out_a = binding.decode_put(a.pool, q, a.table, a.seq_len, M, k_new, v_new,
                               workspace=poisoned_workspace(a, 1, w.q_heads))
    over = torch.tensor([M + 1, INT32_MAX], dtype=torch.int32, device=dev)
    out_b = binding.decode_put(b.pool, q, b.table, over, M, k_new, v_new,
                               workspace=poisoned_workspace(b, 1, w.q_heads))
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all(), "the row went somewhere else than position max_seq_len - 1"
    assert_close(out_a, oracle_from_history(ks, vs, q, [M, M]), "decode_put at max_seq_len")
