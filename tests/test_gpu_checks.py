"""GPU tests of the optional host validation (environment variable KVP_CHECK=1, the conventions
of include/kvpaged.h): every call copies the device lengths, table entries or page ids to the
host first and refuses bad ones with KV_E_ARG before any launch, so the output and the pool
keep every byte; good calls give the same bytes as without the check.  A length below the
call's row count is allowed (its rows at negative positions see no key and get zeros).

The first test establishes that the check is active with a refusal that would be harmless
without it (a page id outside the pool is never dereferenced); the length cases that rely on
the check come after it.
"""
import pytest
import torch

from gpu_support import assert_close, attend, new_cache, oracle_for, pool_bits, say
from paged_kv_cache_rows_amd import binding, workloads

pytestmark = pytest.mark.gpu

KV_E_ARG = -1


def _w(**kw):
    base = dict(name="t", streams=3, kv_heads=2, group=8, head_dim=128, page_size=64, rows=1,
                lengths=[700, 97, 300], spare_frac=0.2, min_spares=2, seed=31)
    base.update(kw)
    return workloads.Workload(**base)


def _refused(fn, what):
    with pytest.raises(binding.KvError) as e:
        fn()
    assert e.value.status == KV_E_ARG, f"{what}: {e.value}"
    return str(e.value)


def _sentinel_out(q):
    return torch.full_like(q.view(torch.int16), 0x5A5A).view(torch.bfloat16)


@pytest.mark.parametrize("entry,R,G", [("decode", 1, 8), ("verify", 4, 8), ("prefill", 64, 4)])
def test_checked_calls_refuse_bad_table_entries_and_lengths(entry, R, G, monkeypatch):
    w = _w(rows=R, group=G)
    say(f"KVP_CHECK {entry} R={R} G={G}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    plain = attend(entry, c, q)

    monkeypatch.setenv("KVP_CHECK", "1")
    checked = attend(entry, c, q)
    assert torch.equal(plain.view(torch.int16), checked.view(torch.int16))

    # a table entry outside the pool inside stream 1's pages (97 keys: entries 0 and 1)
    good_table = c.table.clone()
    c.table[1, 1] = c.pool.num_pages
    out = _sentinel_out(q)
    msg = _refused(lambda: attend(entry, c, q, out=out), "entry outside the pool")
    assert "table entry" in msg
    c.table[1, 1] = -7
    _refused(lambda: attend(entry, c, q, out=out), "negative entry")
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0x5A5A).all(), "a refused call wrote its output"
    # entries past a stream's pages are not read and not checked
    c.table.copy_(good_table)
    c.table[1, 2:] = -1
    again = attend(entry, c, q)
    assert torch.equal(plain.view(torch.int16), again.view(torch.int16))

    # lengths: above max_seq_len, and negative, refused; the output keeps every byte
    good_len = c.seq_len.clone()
    c.seq_len[2] = c.max_seq_len + 1
    msg = _refused(lambda: attend(entry, c, q, out=out), "length above max_seq_len")
    assert "seq_len" in msg
    c.seq_len[2] = -1
    _refused(lambda: attend(entry, c, q, out=out), "negative length")
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0x5A5A).all(), "a refused call wrote its output"
    c.seq_len.copy_(good_len)


@pytest.mark.parametrize("entry,R,G", [("decode", 1, 8), ("verify", 4, 8), ("prefill", 64, 4)])
def test_checked_calls_accept_streams_shorter_than_their_rows(entry, R, G, monkeypatch):
    lengths = [700, 0, max(1, R - 2)]
    w = _w(rows=R, group=G, lengths=lengths)
    say(f"KVP_CHECK short streams {entry} R={R}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    plain = attend(entry, c, q)
    monkeypatch.setenv("KVP_CHECK", "1")
    checked = attend(entry, c, q)
    assert torch.equal(plain.view(torch.int16), checked.view(torch.int16))
    assert (checked[1].view(torch.int16) == 0).all()
    assert_close(checked, oracle_for(c, q), f"{entry} short streams under KVP_CHECK")


def test_checked_row_write_refuses_bad_tables_and_keeps_the_pool(monkeypatch):
    w = _w(rows=3)
    c, _, _ = new_cache(w)
    kn = workloads.normal_bf16((w.streams, 3, w.kv_heads, w.head_dim), 501).cuda()
    vn = workloads.normal_bf16((w.streams, 3, w.kv_heads, w.head_dim), 502).cuda()
    monkeypatch.setenv("KVP_CHECK", "1")
    before = pool_bits(c)
    c.table[0, 3] = c.pool.num_pages + 5
    _refused(lambda: binding.rows_put(c.pool, c.table, c.seq_len, kn, vn, c.max_seq_len), "rows_put entry")
    c.table[0, 3] = int(c.table_host[0, 3])
    c.seq_len[1] = c.max_seq_len + 3
    _refused(lambda: binding.rows_put(c.pool, c.table, c.seq_len, kn, vn, c.max_seq_len), "rows_put length")
    torch.cuda.synchronize()
    after = pool_bits(c)
    assert (before[0] == after[0]).all() and (before[1] == after[1]).all(), "a refused row write changed the pool"


def test_checked_page_copy_refuses_overlaps_and_duplicates(monkeypatch):
    w = _w()
    c, _, _ = new_cache(w)
    monkeypatch.setenv("KVP_CHECK", "1")
    before = pool_bits(c)
    free = [int(x) for x in c.table_host[0, :4]]
    dev = lambda xs: torch.tensor(xs, dtype=torch.int32, device="cuda")
    msg = _refused(lambda: binding.pages_copy(c.pool, dev(free[:2]), dev([free[2], free[2]])), "duplicate destination")
    assert "destination twice" in msg
    msg = _refused(lambda: binding.pages_copy(c.pool, dev(free[:2]), dev([free[1], free[3]])), "source as destination")
    assert "both a source and a destination" in msg
    _refused(lambda: binding.pages_copy(c.pool, dev([free[0]]), dev([c.pool.num_pages])), "id outside the pool")
    torch.cuda.synchronize()
    after = pool_bits(c)
    assert (before[0] == after[0]).all() and (before[1] == after[1]).all(), "a refused copy changed the pool"
