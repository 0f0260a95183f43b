"""GPU parity tests at head dim 256 (the head-dim-256 twins of TensorFold PR #1620's merge
discussion), through the C ABI: decode and short verify windows on the VALU kernel (two lanes
per key in the score, two key rows per load), longer windows, draft trees and prompt chunks on
the MFMA kernel (32-key tiles), sliding windows and rings, the fused row write, pages of 1, 37,
64 and 512, and byte-equality under another page order and an identity table.
"""
import numpy as np
import pytest
import torch

from gpu_support import (assert_close, attend, new_cache, oracle_for, oracle_from_history, oracle_tree_for,
                         poisoned_workspace, pool_bits, random_tree_masks, say)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu

D = 256


def _w(G, R, P, lengths, Hkv=2, window=0, ring=0, seed=256):
    return workloads.Workload(name="d256", streams=len(lengths), kv_heads=Hkv, group=G, head_dim=D, page_size=P,
                              rows=R, lengths=lengths, window=window, ring_pages=ring, spare_frac=0.15,
                              min_spares=2, seed=seed)


def _entry(R):
    return "decode" if R == 1 else ("verify" if R <= 8 else "prefill")


@pytest.mark.parametrize("G,R", [(4, 1), (8, 1), (12, 1), (4, 2), (4, 3), (8, 2), (8, 4), (8, 8), (12, 2),
                                 (16, 1), (16, 4), (4, 64)])
@pytest.mark.parametrize("P", [37, 64, 512])
def test_head_dim_256_matches_the_oracle(G, R, P):
    Hkv = 1 if G >= 12 else 2
    w = _w(G, R, P, [3000, 517, R, 64 * 9 + 5], Hkv=Hkv)
    say(f"d256 G={G} R={R} P={P} ({'VALU' if R * G < 16 else 'MFMA'})")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend(_entry(R), c, q)
    assert_close(out, oracle_for(c, q), f"d256 G={G} R={R} P={P}")
    # the same bytes under another page order and under an identity table
    c2, _, _ = new_cache(w, order_seed=991)
    assert torch.equal(out.view(torch.int16), attend(_entry(R), c2, q).view(torch.int16))
    c3, _, _ = new_cache(w, identity=True)
    assert torch.equal(out.view(torch.int16), attend(_entry(R), c3, q).view(torch.int16))


@pytest.mark.parametrize("G,R", [(8, 1), (4, 3), (8, 4), (16, 2)])
def test_head_dim_256_at_pages_of_one(G, R):
    w = _w(G, R, 1, [700, 33], Hkv=1)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q), oracle_for(c, q), f"d256 P=1 G={G} R={R}")


@pytest.mark.parametrize("G,R", [(8, 1), (4, 2), (8, 4), (8, 8)])
@pytest.mark.parametrize("window,ring", [(1, 0), (100, 0), (1000, 0), (700, 13)])
def test_head_dim_256_sliding_windows_and_rings(G, R, window, ring):
    w = _w(G, R, 64, [2500, 800, R + 5], window=window, ring=ring)
    say(f"d256 window {window} ring {ring} G={G} R={R}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q, window=window), oracle_for(c, q, window), f"d256 W={window} ring={ring}")


@pytest.mark.parametrize("G,R", [(4, 3), (8, 4), (8, 8)])
def test_head_dim_256_draft_trees(G, R):
    w = _w(G, R, 37, [1900, 400, R])
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(G * 10 + R), w.streams, R)
    m = torch.tensor(masks, dtype=torch.int32, device=c.table.device)
    out = binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, m,
                              workspace=poisoned_workspace(c, R, w.q_heads))
    torch.cuda.synchronize()
    assert_close(out, oracle_tree_for(c, q, masks), f"d256 tree G={G} R={R}")


def test_head_dim_256_prompt_in_chunks_equals_one_call():
    w = _w(4, 256, 64, [1024], Hkv=2)
    c, ks, vs = new_cache(w)
    q = workloads.normal_bf16((1, 1024, w.q_heads, D), 2561).cuda()
    whole = binding.prefill(c.pool, q, c.table, c.seq_len, 1024)
    parts = []
    for c0 in range(0, 1024, 256):
        seq = torch.tensor([c0 + 256], dtype=torch.int32, device="cuda")
        parts.append(binding.prefill(c.pool, q[:, c0:c0 + 256].contiguous(), c.table, seq, 1024))
    torch.cuda.synchronize()
    ref = oracle_from_history(ks, vs, q, [1024])
    assert_close(whole, ref, "d256 prompt, one call")
    assert_close(torch.cat(parts, dim=1), ref, "d256 prompt in chunks")


@pytest.mark.parametrize("G", [4, 8, 16])
def test_head_dim_256_decode_put_equals_rows_put_then_decode(G):
    lengths = [2049, 512, 1]
    w = _w(G, 1, 37, lengths, Hkv=1 if G == 16 else 2)
    order = workloads.free_order(w.pool_pages, 2562)
    ks, vs = workloads.kv_history(w)
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=[L - 1 for L in lengths])
        caches.append(c)
    a, b = caches
    dev = a.table.device
    k_new = torch.stack([ks[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    v_new = torch.stack([vs[s][L - 1:L] for s, L in enumerate(lengths)]).to(dev).contiguous()
    q = workloads.queries(w).cuda()
    ml = max(lengths)
    binding.rows_put(a.pool, a.table, a.seq_len, k_new, v_new, ml)
    out_a = binding.decode(a.pool, q, a.table, a.seq_len, ml, workspace=poisoned_workspace(a, 1, w.q_heads))
    out_b = binding.decode_put(b.pool, q, b.table, b.seq_len, ml, k_new, v_new,
                               workspace=poisoned_workspace(b, 1, w.q_heads))
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all()
    assert_close(out_b, oracle_from_history(ks, vs, q, lengths), f"d256 decode_put G={G}")


@pytest.mark.parametrize("R", [1, 4])
def test_head_dim_256_long_stream(R):
    w = _w(8, R, 512, [40960, 33000], Hkv=4)
    say(f"d256 long streams R={R}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q), oracle_for(c, q), f"d256 40k R={R}")
