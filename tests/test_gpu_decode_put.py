"""GPU tests of paged_attn_decode_put: the row write of kv_rows_put fused into the decode
(TensorFold PR #1620, opening description: the new K/V row is written into the pages, then
attention reads through the table).  Two caches with the same pages and history get the new
row, one through kv_rows_put + paged_attn_decode, the other through the fused call: the
outputs and every byte of the two pools must be equal, and the output must match the oracle.
"""
import pytest
import torch

from gpu_support import assert_close, oracle_from_history, pool_bits, poisoned_workspace, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _w(P, D, G, lengths, window=0, ring=0):
    return workloads.Workload(name="put", streams=len(lengths), kv_heads=2 if D == 128 else 1, group=G, head_dim=D,
                              page_size=P, rows=1, lengths=lengths, window=window, ring_pages=ring, spare_frac=0.2,
                              min_spares=2, seed=81)


def _new_rows(ks, vs, lengths, dev):
    k = torch.stack([ks[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    v = torch.stack([vs[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    return k, v


@pytest.mark.parametrize("P,D,G,lengths,window,ring", [
    (64, 128, 8, [300, 129, 1], 0, 0),
    (37, 128, 4, [2048, 2049, 111], 0, 0),
    (512, 128, 8, [1023, 1024, 1025], 0, 0),
    (1, 128, 4, [7, 2, 1], 0, 0),
    (37, 512, 8, [900, 38], 0, 0),
    (64, 128, 8, [1000, 300], 100, 2),
    (64, 128, 4, [3000, 700], 64, 0),
])
def test_decode_put_equals_rows_put_then_decode(P, D, G, lengths, window, ring):
    w = _w(P, D, G, lengths, window, ring)
    say(f"decode_put P={P} D={D} G={G} L={lengths} window={window} ring={ring}")
    order = workloads.free_order(w.pool_pages, 8101)
    ks, vs = workloads.kv_history(w)
    before = [L - 1 for L in lengths]
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=before)
        caches.append(c)
    dev = caches[0].table.device
    k_new, v_new = _new_rows(ks, vs, lengths, dev)
    q = workloads.queries(w).cuda()
    ml = max(lengths)
    a, b = caches
    binding.rows_put(a.pool, a.table, a.seq_len, k_new, v_new, ml, ring_pages=a.ring_pages)
    out_a = binding.decode(a.pool, q, a.table, a.seq_len, ml, window=window, ring_pages=a.ring_pages,
                           workspace=poisoned_workspace(a, 1, w.q_heads, window))
    out_b = binding.decode_put(b.pool, q, b.table, b.seq_len, ml, k_new, v_new, window=window,
                               ring_pages=b.ring_pages, workspace=poisoned_workspace(b, 1, w.q_heads, window))
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "fused output differs"
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all(), "fused row write left different pool bytes"
    assert_close(out_b, oracle_from_history(ks, vs, q, lengths, window), f"decode_put P={P} D={D}")


def test_decode_put_replayed_in_a_graph_as_streams_grow():
    w = _w(64, 128, 8, [900, 403, 1500])
    steps = 3
    ks, vs = workloads.kv_history(w)
    start = [L - steps for L in w.lengths]
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 8102))
    staging.write_history(c, ks, vs, upto=[L - 1 for L in start])
    dev = c.table.device
    ml = max(w.lengths)
    seq = torch.tensor(start, dtype=torch.int32, device=dev)
    k_new, v_new = _new_rows(ks, vs, start, dev)
    q = workloads.normal_bf16((w.streams, 1, w.q_heads, w.head_dim), 811).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(binding.workspace_size(c.pool, c.table, seq, 1, w.q_heads, ml), dtype=torch.uint8, device=dev)

    def step(o):
        binding.decode_put(c.pool, q, c.table, seq, ml, k_new, v_new, out=o, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)                           # writes row start - 1
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()
    for i in range(steps):
        lengths = [L0 + i + 1 for L0 in start]
        say(f"decode_put replay {i}: lengths {lengths}")
        seq.copy_(torch.tensor(lengths, dtype=torch.int32))
        kn, vn = _new_rows(ks, vs, lengths, dev)
        k_new.copy_(kn)
        v_new.copy_(vn)
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = torch.empty_like(q)
        step(eager)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs from eager"
        assert_close(got, oracle_from_history(ks, vs, q, lengths), f"replay {i}")
    del g
