"""GPU tests of paged_attn_prefill_put: the row write of a prompt chunk fused into the prefill
(TensorFold PR #1620, opening description, Writes and Reads bullets: the chunk's K/V rows are
written into the pages, then attention reads through the table).  Two caches with the same
pages and history get the chunk's rows, one through kv_rows_put + paged_attn_prefill, the other
through the fused call: the outputs and every byte of the two pools must be equal, and the
output must match the oracle.  The fused launch runs at head_dim 128 over pages of a multiple
of 64 positions (direct and split plans); the other shapes take the two-launch form.
"""
import pytest
import torch

from gpu_support import assert_close, oracle_from_history, pool_bits, poisoned_workspace, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _w(P, D, G, Hkv, lengths, R, window=0, ring=0, seed=91):
    return workloads.Workload(name="pput", streams=len(lengths), kv_heads=Hkv, group=G, head_dim=D, page_size=P,
                              rows=R, lengths=lengths, window=window, ring_pages=ring, spare_frac=0.2, min_spares=2,
                              seed=seed)


def _chunk_rows(ks, vs, lengths, R, dev):
    """k_new / v_new [S][R][Hkv][D]: the rows at positions L - R .. L - 1 (zeros before 0)."""
    def rows(xs):
        out = []
        for s, L in enumerate(lengths):
            x = xs[s][max(L - R, 0):L]
            if L < R:
                x = torch.cat([torch.zeros((R - L,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device), x])
            out.append(x)
        return torch.stack(out).to(dev).contiguous()
    return rows(ks), rows(vs)


def _both(w, lengths, R, window, order_seed, qseed):
    """Two caches with the history before the chunk; the chunk through the two calls and
    through the fused call.  Returns (out two calls, out fused, caches, history, queries)."""
    order = workloads.free_order(w.pool_pages, order_seed)
    ks, vs = workloads.kv_history(w)
    before = [max(L - R, 0) for L in lengths]
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=before)
        caches.append(c)
    a, b = caches
    dev = a.table.device
    k_new, v_new = _chunk_rows(ks, vs, lengths, R, dev)
    q = workloads.normal_bf16((w.streams, R, w.q_heads, w.head_dim), qseed).to(dev)
    ml = max(lengths)
    binding.rows_put(a.pool, a.table, a.seq_len, k_new, v_new, ml, ring_pages=a.ring_pages)
    out_a = binding.prefill(a.pool, q, a.table, a.seq_len, ml, window=window, ring_pages=a.ring_pages,
                            workspace=poisoned_workspace(a, R, w.q_heads, window))
    out_b = binding.prefill_put(b.pool, q, b.table, b.seq_len, ml, k_new, v_new, window=window,
                                ring_pages=b.ring_pages, workspace=poisoned_workspace(b, R, w.q_heads, window))
    torch.cuda.synchronize()
    return out_a, out_b, caches, ks, vs, q


@pytest.mark.parametrize("P,D,G,Hkv,lengths,R,window,ring", [
    (512, 128, 4, 8, [2048], 512, 0, 0),              # a 512-row prompt chunk: the direct plan
    (64, 128, 4, 2, [1024, 700], 256, 0, 0),          # split plan over 64-key pages
    (64, 128, 8, 2, [3000, 129, 640], 64, 0, 0),      # ragged streams
    (64, 128, 12, 1, [900, 333], 40, 0, 0),           # group 12: tiles cut rows
    (512, 128, 16, 1, [4000], 1, 0, 0),               # one row, MFMA (decode-shaped)
    (64, 128, 4, 2, [100, 300], 128, 0, 0),           # rows before position 0
    (512, 128, 4, 2, [2048, 1600], 512, 1024, 3),     # window 1024 on a 3-page ring
    (37, 128, 4, 2, [900, 500], 64, 0, 0),            # pages of 37: two launches
    (512, 256, 8, 2, [1500], 32, 0, 0),               # head_dim 256: two launches
    (64, 128, 4, 2, [700, 65], 3, 0, 0),              # VALU with 3 rows: two launches
    (64, 128, 4, 2, [700, 65], 1, 0, 0),              # VALU with one row: one launch
])
def test_prefill_put_equals_rows_put_then_prefill(P, D, G, Hkv, lengths, R, window, ring):
    say(f"prefill_put P={P} D={D} G={G} Hkv={Hkv} L={lengths} R={R} window={window} ring={ring}")
    w = _w(P, D, G, Hkv, lengths, R, window, ring)
    out_a, out_b, (a, b), ks, vs, q = _both(w, lengths, R, window, 9101, 911)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), "fused output differs"
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all(), "fused row write left different pool bytes"
    assert_close(out_b, oracle_from_history(ks, vs, q, lengths, window), f"prefill_put P={P} D={D} R={R}")


@pytest.mark.parametrize("window,ring", [(0, 0), (1024, 3)])
def test_chunked_prompt_through_prefill_put(window, ring):
    """A 2,048-token prompt in four 512-row chunks, each through the fused call, on one cache:
    every chunk matches the oracle, and the pool ends byte-equal to the two-call prompt."""
    say(f"chunked prefill_put window={window} ring={ring}")
    w = workloads.prefill_mixed(window=window)
    order = workloads.free_order(w.pool_pages, 9102)
    ks, vs = workloads.kv_history(w)
    caches = [staging.make_cache(w, order=order, lengths=[2048]) for _ in range(2)]
    a, b = caches
    dev = a.table.device
    qa = workloads.normal_bf16((1, 2048, w.q_heads, w.head_dim), 912).to(dev)
    for c0 in range(0, 2048, 512):
        seq_a = torch.tensor([c0 + 512], dtype=torch.int32, device=dev)
        seq_b = seq_a.clone()
        kn = ks[0][c0:c0 + 512][None].to(dev).contiguous()
        vn = vs[0][c0:c0 + 512][None].to(dev).contiguous()
        q = qa[:, c0:c0 + 512].contiguous()
        binding.rows_put(a.pool, a.table, seq_a, kn, vn, 2048, ring_pages=a.ring_pages)
        out_a = binding.prefill(a.pool, q, a.table, seq_a, 2048, window=window, ring_pages=a.ring_pages)
        out_b = binding.prefill_put(b.pool, q, b.table, seq_b, 2048, kn, vn, window=window, ring_pages=b.ring_pages)
        torch.cuda.synchronize()
        assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16)), f"chunk at {c0} differs"
        assert_close(out_b, oracle_from_history(ks, vs, q, [c0 + 512], window), f"chunk at {c0}")
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all(), "pools differ after the prompt"


def test_prefill_put_refuses_null_rows():
    w = _w(64, 128, 4, 2, [300], 32)
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 9103))
    q = workloads.normal_bf16((1, 32, w.q_heads, 128), 913).cuda()
    k_new = torch.zeros((1, 32, 2, 128), dtype=torch.bfloat16, device="cuda")
    lay = binding._layout(c.pool, c.table, c.seq_len, 32, 300, 0)
    out = torch.empty_like(q)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    args = binding.AttnArgs(binding._ptr(q), binding._ptr(out), w.q_heads, 0.0, 0, binding._ptr(ws), ws.numel())
    import ctypes
    rc = binding.load().paged_attn_prefill_put(c.pool.handle, ctypes.byref(lay), ctypes.byref(args),
                                               binding._ptr(k_new), None, None)
    assert rc == -1, rc
