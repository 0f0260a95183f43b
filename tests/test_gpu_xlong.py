"""GPU parity tests at large sizes and high addresses.

* One stream of 262,144 keys: decode on the VALU path and a 4-row verify on the MFMA path, with
  hundreds of splits.
* A stream whose pages all have ids above 65,536 in a pool of 70,000 pages (ids that do not fit
  16 bits).
* Pools larger than 2^31 elements per operand (4 GiB of bf16 each for K and V): the stream's
  pages sit at the top of the pool, so every element offset the kernels form exceeds 2^31 and
  would wrap in 32-bit arithmetic.  Decode (VALU), verify (MFMA), a prompt chunk, the row
  write and the fused row write + decode are compared with the oracle, at the headline geometry
  (pages of 512, one lookup per tile) and at head dim 512 over pages of 37 (lookups per row).

Every output is compared in full with the oracle.  The long stream's pool is also compared byte
for byte with the oracle's scatter of its history before it is attended, so that a wrong
output can be told apart from wrong pages.
"""
import numpy as np
import pytest
import torch

from gpu_support import (assert_close, attend, expected_pool, oracle_for, oracle_from_history, pool_bits, remember,
                         say)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu

LONG = 262144


def _long(P, rows):
    return workloads.Workload(name="long", streams=1, kv_heads=1, group=8, head_dim=128, page_size=P, rows=rows,
                              lengths=[LONG], spare_frac=0.02, min_spares=2, seed=91)


def _pool_is_the_history(c):
    kb, vb = expected_pool(c)
    ka, va = pool_bits(c)
    bad_k = np.argwhere((ka != kb).any(axis=(1, 2, 3))).ravel()
    bad_v = np.argwhere((va != vb).any(axis=(1, 2, 3))).ravel()
    assert bad_k.size == 0 and bad_v.size == 0, f"pages differing from the oracle's scatter: K {bad_k[:8]}, V {bad_v[:8]}"


@pytest.mark.parametrize("P", [64, 37])
def test_decode_over_262144_keys(P):
    w = _long(P, 1)
    say(f"decode over {LONG} keys, pages of {P}, pool {w.pool_pages}")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 9101))
    ks, vs = workloads.kv_history(w)
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    _pool_is_the_history(c)
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
    remember(c, ks, vs)
    _pool_is_the_history(c)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q)
    again = attend("verify", c, q)
    assert torch.equal(out.view(torch.int16), again.view(torch.int16)), "a repeat of the call gave other bytes"
    assert_close(out, oracle_for(c, q), f"verify R=4 L={LONG}")


def test_pages_with_ids_above_65536():
    # 1,250 pages of 16 at the top of a 70,000-page pool
    w = workloads.Workload(name="high_ids", streams=1, kv_heads=1, group=8, head_dim=128, page_size=16, rows=1,
                           lengths=[20000], spare_frac=55.0, min_spares=2, seed=92)
    assert w.pool_pages == 70000
    order = np.arange(w.pool_pages, dtype=np.int32)[::-1].copy()
    say(f"pages with high ids: pool {w.pool_pages}")
    c = staging.make_cache(w, order=order)
    assert c.table_host[0][:w.pages_for(20000)].min() > 65536
    ks, vs = workloads.kv_history(w)
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    for rows, mode in ((1, "decode"), (4, "verify")):
        q = workloads.queries(w, rows=rows, salt=rows).cuda()
        out = attend(mode, c, q)
        assert_close(out, oracle_for(c, q), f"{mode} on pages above 65536")


@pytest.mark.parametrize("kv_heads,group,D,P,L", [(8, 8, 128, 512, 20000), (1, 8, 512, 37, 9000)])
def test_pool_beyond_2_31_elements(kv_heads, group, D, P, L):
    page_elems = kv_heads * P * D
    used = -(-L // P)
    # the first used page starts past element 2^31, and the pool ends a few pages after the last
    first = (1 << 31) // page_elems + 1
    num_pages = first + used + 3
    assert first * page_elems > (1 << 31) and num_pages * page_elems * 2 * 2 < (20 << 30)
    w = workloads.Workload(name="beyond_2_31", streams=1, kv_heads=kv_heads, group=group, head_dim=D,
                           page_size=P, rows=1, lengths=[L], spare_frac=0.0, min_spares=0, seed=93)
    say(f"pool of {num_pages} pages x {page_elems} elements ({num_pages * page_elems / 2 ** 31:.2f} x 2^31 per "
        f"operand), stream of {L} keys at pages {first}..{first + used - 1}, D={D} P={P}")
    # hand out the top pages first, in a shuffled order
    top = np.arange(first, first + used, dtype=np.int32)
    rest = np.setdiff1d(np.arange(num_pages, dtype=np.int32), top)
    order = np.concatenate([np.random.default_rng(931).permutation(top), rest]).astype(np.int32)
    pool = binding.Pool(num_pages, P, kv_heads, D, max_streams=1, free_order=order)
    ids = pool.lease(0, used)
    assert min(ids) * page_elems > (1 << 31)
    dev = pool.k_pages.device
    table = torch.tensor([ids], dtype=torch.int32, device=dev)
    ks, vs = workloads.kv_history(w)
    # the prompt: all rows but the last 8 in chunks through kv_rows_put, then a 512-row-or-less
    # prompt chunk attended, then the last rows through the fused row write + decode
    head = L - 8
    for c0 in range(0, head, 4096):
        c1 = min(head, c0 + 4096)
        binding.rows_put(pool, table, torch.tensor([c1], dtype=torch.int32, device=dev),
                         ks[0][c0:c1][None].contiguous().to(dev), vs[0][c0:c1][None].contiguous().to(dev), c1)
    R = min(256, head)
    qp = workloads.normal_bf16((1, R, w.q_heads, D), 932).to(dev)
    seq = torch.tensor([head], dtype=torch.int32, device=dev)
    outp = binding.prefill(pool, qp, table, seq, L)
    torch.cuda.synchronize()
    assert_close(outp, oracle_from_history(ks, vs, qp, [head]), f"prompt chunk of {R} rows at {head}")
    for i in range(head, L):
        seq = torch.tensor([i + 1], dtype=torch.int32, device=dev)
        qd = workloads.normal_bf16((1, 1, w.q_heads, D), 940 + i - head).to(dev)
        out = binding.decode_put(pool, qd, table, seq, L, ks[0][i:i + 1][None].contiguous().to(dev),
                                 vs[0][i:i + 1][None].contiguous().to(dev))
        torch.cuda.synchronize()
        assert_close(out, oracle_from_history(ks, vs, qd, [i + 1]), f"decode_put at {i + 1}")
    seq = torch.tensor([L], dtype=torch.int32, device=dev)
    qv = workloads.normal_bf16((1, 4, w.q_heads, D), 950).to(dev)
    outv = binding.verify(pool, qv, table, seq, L)
    qd = workloads.normal_bf16((1, 1, w.q_heads, D), 951).to(dev)
    outd = binding.decode(pool, qd, table, seq, L)
    torch.cuda.synchronize()
    assert_close(outv, oracle_from_history(ks, vs, qv, [L]), "verify 4 rows")
    assert_close(outd, oracle_from_history(ks, vs, qd, [L]), "decode")
    # the rows landed where the table says: the stream's last page holds its last rows, and the
    # pages below `first` were never written
    last = ids[(L - 1) // P]
    n_last = L - ((L - 1) // P) * P
    got = pool.k_pages[last, :, :n_last].cpu()
    want = ks[0][L - n_last:L].transpose(0, 1)
    assert torch.equal(got.view(torch.int16), want.contiguous().view(torch.int16))
    untouched = pool.k_pages[:first].view(torch.int16)
    assert bool((untouched == workloads.NAN_BITS).all())
    del pool, table
    torch.cuda.empty_cache()
