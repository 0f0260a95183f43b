"""GPU test of paged_attn_decode_put_static, the decode step for callers that cannot allocate:
called through the C ABI, it must give the bytes of paged_attn_decode_put (output and pool)
on two calls in a row, the second smaller than the first (the library's scratch keeps the
first call's partials, which the second must never read), match the oracle, and refuse a call
whose partials do not fit the scratch before launching anything.
"""
import pytest
import torch

from gpu_support import assert_close, oracle_from_history, pool_bits, poisoned_workspace, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _pair(w, order_seed):
    """Two caches with the same pages and the history up to the last row of every stream, and
    the last rows as the step's new rows."""
    order = workloads.free_order(w.pool_pages, order_seed)
    ks, vs = workloads.kv_history(w, device="cuda")
    before = [L - 1 for L in w.lengths]
    caches = []
    for _ in range(2):
        c = staging.make_cache(w, order=order)
        staging.write_history(c, ks, vs, upto=before)
        caches.append(c)
    dev = caches[0].table.device
    k_new = torch.stack([ks[s][L - 1:L] for s, L in enumerate(w.lengths)]).to(dev).contiguous()
    v_new = torch.stack([vs[s][L - 1:L] for s, L in enumerate(w.lengths)]).to(dev).contiguous()
    return caches, ks, vs, k_new, v_new


@pytest.mark.parametrize("big,small", [
    (dict(streams=12, kv_heads=8, group=8, head_dim=128, page_size=512, lengths=[40000, 33000, 36000, 39000,
                                                                                  34567, 40960, 32768, 35000,
                                                                                  38000, 37000, 33333, 39999]),
     dict(streams=3, kv_heads=8, group=8, head_dim=128, page_size=512, lengths=[900, 5000, 1])),
    (dict(streams=4, kv_heads=2, group=8, head_dim=512, page_size=37, lengths=[9000, 2048, 4000, 100]),
     dict(streams=2, kv_heads=2, group=8, head_dim=512, page_size=37, lengths=[2048, 37])),
])
def test_static_scratch_decode_equals_the_workspace_decode(big, small):
    for i, shape in enumerate((big, small)):
        w = workloads.Workload(name="static", rows=1, spare_frac=0.1, min_spares=2, seed=61 + i, **shape)
        say(f"call {i}: {w.streams} streams, D={w.head_dim}, P={w.page_size}, lengths {w.lengths}")
        (a, b), ks, vs, k_new, v_new = _pair(w, 6100 + i)
        q = workloads.queries(w, device="cuda")
        ml = max(w.lengths)
        need = binding.workspace_size(a.pool, a.table, a.seq_len, 1, w.q_heads, ml)
        assert 0 < need <= binding.STATIC_SCRATCH_BYTES
        ref = binding.decode_put(a.pool, q, a.table, a.seq_len, ml, k_new, v_new,
                                 workspace=poisoned_workspace(a, 1, w.q_heads))
        out = torch.full_like(q.view(torch.int16), 0x7FC0).view(torch.bfloat16)
        got = binding.decode_put_static(b.pool, q, b.table, b.seq_len, ml, k_new, v_new, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), f"call {i}: output bytes differ"
        ka, va = pool_bits(a)
        kb, vb = pool_bits(b)
        assert (ka == kb).all() and (va == vb).all(), f"call {i}: pool bytes differ"
        assert_close(got, oracle_from_history(ks, vs, q, w.lengths), f"call {i} against the oracle")
        a.pool.close()
        b.pool.close()
        del a, b
        torch.cuda.empty_cache()


def test_static_scratch_refuses_a_call_that_does_not_fit():
    # 200 streams at a 40k ceiling need about 100 MB of partials: refused before any launch
    S, ml, P = 200, 40960, 512
    pool = binding.Pool(4, P, 8, 128, max_streams=1)
    dev = pool.k_pages.device
    table = torch.zeros((S, ml // P), dtype=torch.int32, device=dev)
    seq = torch.full((S,), ml, dtype=torch.int32, device=dev)
    q = torch.zeros((S, 1, 64, 128), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((S, 1, 8, 128), dtype=torch.bfloat16, device=dev)
    need = binding.workspace_size(pool, table, seq, 1, 64, ml)
    assert need > binding.STATIC_SCRATCH_BYTES
    out = torch.full_like(q.view(torch.int16), 0x5A5A).view(torch.bfloat16)
    before = (workloads.bf16_bits(pool.k_pages), workloads.bf16_bits(pool.v_pages))
    with pytest.raises(binding.KvError) as e:
        binding.decode_put_static(pool, q, table, seq, ml, kn, kn, out=out)
    assert e.value.status == binding.KV_E_WORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out.view(torch.int16) == 0x5A5A).all()
    after = (workloads.bf16_bits(pool.k_pages), workloads.bf16_bits(pool.v_pages))
    assert (before[0] == after[0]).all() and (before[1] == after[1]).all()
