"""GPU parity tests of the row write and the VALU decode / short-verify path, through the C ABI.

Kernel contract after TensorFold PR #1620 (kernel-contract bullet): pages of 512, 37 and 64,
keys shuffled over the pool, NaN in spare pages and in the unused slots of each stream's last
page; checks of repeat (bit-identical reruns), shapes, sums (oracle parity) and nonfinite
values; and a control (the first page id replaced by a spare page's) that must go red.
Plus the linear-vs-paged byte equality of its model test, at kernel level: an identity table
and two shuffled tables give byte-equal outputs.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gpu_support import (assert_close, assert_red, attend, compare, expected_pool, new_cache, oracle_for,
                         oracle_from_history, pool_bits, remember, say)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="t", streams=2, kv_heads=2, group=4, head_dim=128, page_size=64, rows=1,
                lengths=[300, 129], spare_frac=0.2, min_spares=2, seed=7)
    base.update(kw)
    return workloads.Workload(**base)


# ----------------------------------------------------------------------------- row write
@pytest.mark.parametrize("P,D,ring", [(64, 128, 0), (37, 512, 0), (512, 128, 0), (1, 128, 0), (64, 128, 3)])
def test_rows_put_bytes_equal_the_oracle_scatter(P, D, ring):
    say(f"rows_put P={P} D={D} ring={ring}")
    L = 700 if not ring else 1000
    w = _w(page_size=P, head_dim=D, lengths=[L, 333], ring_pages=ring, window=100 if ring else 0)
    c, _, _ = new_cache(w, history=False)
    ks, vs = workloads.kv_history(w)
    rng = np.random.default_rng(P + D)
    shape = (w.pool_pages, w.kv_heads, P, D)
    kbits = np.full(shape, workloads.NAN_BITS, dtype=np.uint16)     # all NaN before any write
    vbits = np.full(shape, workloads.NAN_BITS, dtype=np.uint16)
    gk, gv = pool_bits(c)
    assert np.array_equal(gk, kbits) and np.array_equal(gv, vbits)
    for s, Ls in enumerate(c.lengths):
        pos = 0
        t, _ = c.stream_view(s)
        while pos < Ls:
            R = int(min(rng.integers(1, 150), Ls - pos, ring * P if ring else 10 ** 9))
            pos += R
            seq = torch.tensor([pos], dtype=torch.int32, device="cuda")
            binding.rows_put(c.pool, t, seq, ks[s][pos - R:pos].cuda()[None].contiguous(),
                             vs[s][pos - R:pos].cuda()[None].contiguous(), max_seq_len=pos, ring_pages=ring)
            kbits = oracle.rows_put(kbits, c.table_host[s], pos, workloads.bf16_bits(ks[s][pos - R:pos]), P, ring)
            vbits = oracle.rows_put(vbits, c.table_host[s], pos, workloads.bf16_bits(vs[s][pos - R:pos]), P, ring)
    torch.cuda.synchronize()
    gk, gv = pool_bits(c)
    assert np.array_equal(gk, kbits) and np.array_equal(gv, vbits)


def test_rows_put_batched_streams_and_rows():
    w = _w(lengths=[200, 77], spare_frac=0.0)
    c, ks, vs = new_cache(w)                  # history written stream by stream
    kb0, vb0 = expected_pool(c)               # the oracle's scatter of the same history
    gk, gv = pool_bits(c)
    assert np.array_equal(gk, kb0) and np.array_equal(gv, vb0)
    # overwrite the last 5 rows of both streams in one call with fresh values
    kn = workloads.normal_bf16((2, 5, w.kv_heads, w.head_dim), 99)
    vn = workloads.normal_bf16((2, 5, w.kv_heads, w.head_dim), 98)
    binding.rows_put(c.pool, c.table, c.seq_len, kn.cuda(), vn.cuda(), max_seq_len=c.max_seq_len)
    torch.cuda.synchronize()
    for s in range(2):
        kb0 = oracle.rows_put(kb0, c.table_host[s], c.lengths[s], workloads.bf16_bits(kn[s]), w.page_size)
        vb0 = oracle.rows_put(vb0, c.table_host[s], c.lengths[s], workloads.bf16_bits(vn[s]), w.page_size)
    gk, gv = pool_bits(c)
    assert np.array_equal(gk, kb0) and np.array_equal(gv, vb0)


# ----------------------------------------------------------------------------- tiny decode
def test_tiny_decode_parity_and_contract():
    w = workloads.tiny_decode()
    say(f"tiny decode: pool {w.pool_pages} pages, {w.pages_used} used")
    assert w.pool_pages == 8 and w.pages_used == 5
    c, ks, vs = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("decode", c, q)
    assert out.shape == q.shape
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q), "tiny decode")
    again = attend("decode", c, q)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "repeat is not bit-identical"


@pytest.mark.parametrize("P", [64, 37, 512])
def test_paged_output_is_byte_equal_to_identity_table(P):
    w = _w(page_size=P, lengths=[1500, 2100, 700], streams=3, kv_heads=2, group=8)
    q = workloads.queries(w).cuda()
    outs = []
    for kind in ("identity", 11, 12):
        c, _, _ = new_cache(w, identity=(kind == "identity"), order_seed=None if kind == "identity" else kind)
        if kind == "identity":
            # the identity order hands each stream a contiguous run of pages
            for s in range(3):
                row = c.table_host[s][:w.pages_for(c.lengths[s])]
                assert (np.diff(row) == 1).all()
        outs.append(attend("decode", c, q))
    ref = oracle_for(c, q)
    assert_close(outs[-1], ref, f"decode P={P}")
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16)), "shuffled != identity bytes"


def test_nan_pattern_of_spares_does_not_change_bytes():
    w = _w(lengths=[300, 129])
    q = workloads.queries(w).cuda()
    a = attend("decode", new_cache(w, fill_bits=workloads.NAN_BITS)[0], q)
    b = attend("decode", new_cache(w, fill_bits=workloads.NAN_BITS_ALT)[0], q)
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_control_first_page_id_of_a_spare_goes_red():
    w = workloads.tiny_decode()
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    ref = oracle_for(c, q)
    good = attend("decode", c, q)
    assert compare(good, ref)[0]
    spare = sorted(set(range(w.pool_pages)) - set(c.table_host[0][:w.pages_used].tolist()))[0]
    bad_table = c.table.clone()
    bad_table[0, 0] = spare
    bad = binding.decode(c.pool, q, bad_table, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    assert_red(bad, ref, "a spare page as the first page")


def test_one_key_returns_v_bytes():
    w = _w(lengths=[1, 1], page_size=64, group=8)
    c, ks, vs = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("decode", c, q)
    for s in range(2):
        for h in range(w.q_heads):
            assert torch.equal(out[s, 0, h].cpu().view(torch.int16), vs[s][0, h // w.group].view(torch.int16))


# ----------------------------------------------------------------------------- lengths and pages
@pytest.mark.parametrize("P,lengths", [
    (1, [1, 2, 7]), (3, [5, 64, 65]), (64, [63, 64, 65]), (512, [1023, 1024, 1025]),
    (37, [2048, 2049, 111]), (512, [3000, 4097, 5000]),
])
@pytest.mark.parametrize("D,G", [(128, 8), (128, 4), (512, 8)])
def test_decode_parity_over_lengths_and_pages(P, lengths, D, G):
    w = _w(page_size=P, lengths=lengths, streams=len(lengths), head_dim=D, group=G, kv_heads=2 if D == 128 else 1)
    say(f"decode D={D} G={G} P={P} L={lengths}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("decode", c, q), oracle_for(c, q), f"decode D={D} G={G} P={P}")


@pytest.mark.parametrize("R", [2, 3])
@pytest.mark.parametrize("D", [128, 512])
def test_short_verify_valu_parity(R, D):
    w = _w(rows=R, group=4, head_dim=D, page_size=37, lengths=[900, 40, R], streams=3)
    say(f"verify VALU R={R} D={D}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q)
    assert_close(out, oracle_for(c, q), f"verify R={R} D={D}")
    # each verify row equals a decode at its own length (pages written, rows queried one by one)
    for r in range(R):
        lens = [L - R + r + 1 for L in c.lengths]
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        w1 = dataclasses.replace(w, rows=1)
        one = binding.decode(c.pool, q[:, r:r + 1].contiguous(), c.table, seq, c.max_seq_len)
        torch.cuda.synchronize()
        assert_close(one, oracle_for(c, q[:, r:r + 1].contiguous(), lengths=lens), f"row {r} as decode")


@pytest.mark.parametrize("W", [1, 5, 64, 1000])
def test_sliding_window_decode_full_table(W):
    w = _w(lengths=[3000, 700], window=W, group=8)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("decode", c, q, window=W), oracle_for(c, q, window=W), f"window {W}")


@pytest.mark.parametrize("R", [1, 2, 3])
def test_sliding_window_ring_layer(R):
    W, P, ring = 100, 64, 2            # ring of 128 positions holds window + rows - 1
    w = _w(lengths=[1000, 300], window=W, ring_pages=ring, page_size=P, rows=R, group=4)
    c, ks, vs = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q, window=W)
    assert_close(out, oracle_from_history(ks, vs, q, c.lengths, W), f"ring R={R}")


@pytest.mark.parametrize("S,L", [(40, 3000), (100, 1500)])
def test_decode_many_streams_few_pieces(S, L):
    # many (stream, head) groups: the plan gives each stream 3 pieces (not a multiple of 8) or a
    # single one; sampled streams against the oracle, and a second page order gives the same bytes
    lengths = [L - 13 * (i % 7) for i in range(S)]
    w = workloads.Workload(name="many", streams=S, kv_heads=8, group=8, head_dim=128, page_size=64,
                           rows=1, lengths=lengths, spare_frac=0.05, seed=17)
    say(f"decode {S} streams at about {L} keys")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 501))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    q = workloads.queries(w, device="cuda")
    out = attend("decode", c, q)
    assert_close(out, oracle_for(c, q), f"{S} streams")
    c2 = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 502))
    staging.write_history(c2, ks, vs)
    assert torch.equal(out.view(torch.int16), attend("decode", c2, q).view(torch.int16))


# ----------------------------------------------------------------------------- full-size decode
def test_batched_decode_full_size_all_streams():
    w = workloads.batched_decode()
    say(f"batched decode: lengths {w.lengths}, pool {w.pool_pages} pages")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3002))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    q = workloads.queries(w, device="cuda")
    out = attend("decode", c, q)
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q), "12 streams at 32k-40k keys")
    # a second shuffle of the same cache contents gives the same bytes
    c2 = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 4002))
    staging.write_history(c2, ks, vs)
    out2 = attend("decode", c2, q)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
