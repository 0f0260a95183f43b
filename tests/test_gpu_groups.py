"""GPU parity tests at the head layouts of TensorFold PR #1620's kernel timing (the author's
per-tile follow-up): 48 query heads over 4 KV heads at head dim 128 (GQA group 12) and 16 over 1
at head dim 512 (group 16), at 2k, 9k and 32k keys and 1, 4 and 12 rows, pages of 512 spread
over the pool, plus pages of 37 and 64.  Group 12 decodes on the VALU kernel (12 query vectors)
and verifies on MFMA; group 16 runs MFMA from one row on.  Rows beyond a verify window's 8
run as a prompt chunk.
"""
import pytest
import torch

from gpu_support import assert_close, attend, new_cache, oracle_for, say
from paged_kv_cache_rows_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _w(Hkv, G, D, P, lengths, rows, seed=131):
    return workloads.Workload(name="groups", streams=len(lengths), kv_heads=Hkv, group=G, head_dim=D, page_size=P,
                              rows=rows, lengths=lengths, spare_frac=0.1, min_spares=2, seed=seed)


def _entry(R):
    return "decode" if R == 1 else ("verify" if R <= 8 else "prefill")


@pytest.mark.parametrize("L", [2048, 9000, 32768])
@pytest.mark.parametrize("R", [1, 4, 12])
def test_group_12_at_head_dim_128_the_pages_grid(L, R):
    w = _w(4, 12, 128, 512, [L], R)
    say(f"48/4 heads d128 P512 L={L} R={R} ({'VALU' if R * 12 < 16 else 'MFMA'})")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q), oracle_for(c, q), f"G12 L={L} R={R}")


@pytest.mark.parametrize("L", [9000, 32768])
@pytest.mark.parametrize("R", [1, 4])
def test_group_16_at_head_dim_512_the_pages_grid(L, R):
    w = _w(1, 16, 512, 512, [L], R)
    say(f"16/1 heads d512 P512 L={L} R={R} (MFMA)")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q), oracle_for(c, q), f"G16 L={L} R={R}")


@pytest.mark.parametrize("G,D,Hkv", [(12, 128, 4), (12, 512, 1), (16, 128, 2), (16, 512, 1)])
@pytest.mark.parametrize("P", [37, 64])
@pytest.mark.parametrize("R", [1, 2, 3, 8])
def test_groups_12_and_16_over_odd_pages_and_ragged_streams(G, D, Hkv, P, R):
    w = _w(Hkv, G, D, P, [1500, 300, R, 77], R, seed=132)
    say(f"G={G} D={D} P={P} R={R}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend(_entry(R), c, q)
    assert_close(out, oracle_for(c, q), f"G={G} D={D} P={P} R={R}")
    # byte-equal under another page order, and on a repeat
    c2, _, _ = new_cache(w, order_seed=777)
    assert torch.equal(out.view(torch.int16), attend(_entry(R), c2, q).view(torch.int16))


@pytest.mark.parametrize("G,D,Hkv,R", [(12, 128, 4, 3), (16, 512, 1, 4), (12, 512, 1, 2)])
def test_groups_12_and_16_with_a_sliding_window(G, D, Hkv, R):
    w = _w(Hkv, G, D, 64, [2000, 500], R, seed=133)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q, window=300), oracle_for(c, q, window=300), f"G={G} window 300")


@pytest.mark.parametrize("G,D,Hkv,P", [(16, 512, 1, 512), (16, 128, 2, 37), (12, 128, 4, 64)])
def test_decode_put_at_groups_12_and_16_equals_the_two_calls(G, D, Hkv, P):
    # group 16 decodes on the MFMA kernel, where the row goes in through a row-write launch;
    # group 12 on the VALU kernel, which writes the row itself: both equal kv_rows_put + decode
    from paged_kv_cache_rows_amd import staging
    from gpu_support import oracle_from_history, pool_bits
    w = _w(Hkv, G, D, P, [3000, 700, 1], 1, seed=134)
    say(f"decode_put G={G} D={D} P={P}")
    order = workloads.free_order(w.pool_pages, 1341)
    ks, vs = workloads.kv_history(w)
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=[L - 1 for L in w.lengths])
        caches.append(c)
    a, b = caches
    kn = torch.stack([ks[s][L - 1:L] for s, L in enumerate(w.lengths)]).cuda().contiguous()
    vn = torch.stack([vs[s][L - 1:L] for s, L in enumerate(w.lengths)]).cuda().contiguous()
    q = workloads.queries(w).cuda()
    ml = max(w.lengths)
    binding.rows_put(a.pool, a.table, a.seq_len, kn, vn, ml)
    out_a = binding.decode(a.pool, q, a.table, a.seq_len, ml)
    out_b = binding.decode_put(b.pool, q, b.table, b.seq_len, ml, kn, vn)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    ka, va = pool_bits(a)
    kb, vb = pool_bits(b)
    assert (ka == kb).all() and (va == vb).all()
    assert_close(out_b, oracle_from_history(ks, vs, q, w.lengths), f"decode_put G={G} D={D}")
