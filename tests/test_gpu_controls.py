"""Controls that must go red, at the headline size (12 streams, 32k-40k keys each).

TensorFold PR #1620: the kernel contract checks repeat, shapes, sums and nonfinite values, and
a control (the first page id replaced by a spare page's) must go red; after the per-tile
change the author reports the contract's controls all going red.  Each control here plants one
plausible kernel mistake on the host side, with every access inside the pool, runs the real
kernels on it, and asserts that the parity check against the oracle fails for it, while the
unplanted run (and, where the mistake is local to one stream, the other streams of the planted
run) passes the same check.  The planted mistakes:

1. one table entry of the longest stream pointed at another page of the same stream (a wrong
   per-tile page lookup);
2. one stream's length one too long, with max_seq_len raised to match (an off-by-one length:
   the extra key is an unused slot holding the NaN pattern);
3. the partly filled last page of one stream dropped (a kernel that forgets the ragged tail);
4. the query heads permuted so that the kernels compute the interleaved GQA mapping
   (query head h reading KV head h mod Hkv instead of h div G);
5. K and V swapped (operands crossed);
6. a wrong softmax scale (1/d instead of 1/sqrt(d));
7. the first page id of one stream replaced by a spare page's (the pages' own control).
"""
import numpy as np
import pytest
import torch

from gpu_support import assert_close, assert_red, attend, compare, oracle_for, remember, say
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def headline():
    w = workloads.batched_decode()
    say(f"controls on the batched decode: lengths {w.lengths}")
    c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, 3002))
    ks, vs = workloads.kv_history(w, device="cuda")
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    del ks, vs
    q = workloads.queries(w, device="cuda")
    ref = oracle_for(c, q)
    good = attend("decode", c, q)
    assert_close(good, ref, "unplanted run")
    yield w, c, q, ref
    c.pool.close()
    del c
    torch.cuda.empty_cache()


def _others(ref, out, s, what):
    keep = [i for i in range(ref.shape[0]) if i != s]
    assert_close(out[keep], ref[keep], f"{what}: the other streams")


def test_control_table_entry_pointed_at_another_page_of_the_stream(headline):
    w, c, q, ref = headline
    s = int(np.argmax(c.lengths))
    i = 30
    bad = c.table.clone()
    bad[s, i] = int(c.table_host[s][i + 1])
    out = binding.decode(c.pool, q, bad, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    assert_red(out[s:s + 1], ref[s:s + 1], f"stream {s} entry {i} -> its page {i + 1}")
    assert_red(out, ref, "the same, whole output")
    _others(ref, out, s, "table entry")


def test_control_length_one_too_long(headline):
    w, c, q, ref = headline
    s = next(i for i, L in enumerate(c.lengths) if L % w.page_size != 0)
    seq = c.seq_len.clone()
    seq[s] += 1
    out = binding.decode(c.pool, q, c.table, seq, c.max_seq_len + 1)
    torch.cuda.synchronize()
    assert not torch.isfinite(out[s].float()).all(), "the key past the stream was not read"
    assert_red(out[s:s + 1], ref[s:s + 1], f"stream {s} length {c.lengths[s]} + 1")
    _others(ref, out, s, "length + 1")


def test_control_ragged_last_page_dropped(headline):
    w, c, q, ref = headline
    s = max(range(w.streams), key=lambda i: c.lengths[i] % w.page_size)
    tail = c.lengths[s] % w.page_size
    assert tail > 100
    seq = c.seq_len.clone()
    seq[s] -= tail
    out = binding.decode(c.pool, q, c.table, seq, c.max_seq_len)
    torch.cuda.synchronize()
    assert_red(out[s:s + 1], ref[s:s + 1], f"stream {s}: last {tail} keys dropped")
    _others(ref, out, s, "ragged tail")


def test_control_interleaved_gqa_mapping(headline):
    w, c, q, ref = headline
    Hkv, G = w.kv_heads, w.group
    # query head h placed where the kernels' contiguous mapping reads KV head h mod Hkv
    perm = torch.tensor([(h % Hkv) * G + h // Hkv for h in range(w.q_heads)], device=q.device)
    qp = torch.empty_like(q)
    qp[:, :, perm] = q
    outp = binding.decode(c.pool, qp.contiguous(), c.table, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    out = outp[:, :, perm].contiguous()
    assert_red(out, ref, "interleaved GQA mapping")
    # the permutation itself is sound: heads 0, 9, 18, ... keep their KV head under both maps
    same = [h for h in range(w.q_heads) if h // G == h % Hkv]
    assert_close(out[:, :, same].contiguous(), ref[:, :, same], "heads the two mappings agree on")


def test_control_k_and_v_swapped(headline):
    w, c, q, ref = headline
    crossed = binding.Pool(w.pool_pages, w.page_size, w.kv_heads, w.head_dim, max_streams=w.streams,
                           k_pages=c.pool.v_pages, v_pages=c.pool.k_pages)
    out = binding.decode(crossed, q, c.table, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    crossed.close()
    assert_red(out, ref, "K and V swapped")


def test_control_wrong_scale(headline):
    w, c, q, ref = headline
    out = attend("decode", c, q, scale=1.0 / w.head_dim)
    assert_red(out, ref, "scale 1/d")


def test_control_first_page_a_spare(headline):
    w, c, q, ref = headline
    used = set(int(x) for s, L in enumerate(c.lengths) for x in c.table_host[s][:w.pages_for(L)])
    spare = min(set(range(w.pool_pages)) - used)
    s = 4
    bad = c.table.clone()
    bad[s, 0] = spare
    out = binding.decode(c.pool, q, bad, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    assert_red(out[s:s + 1], ref[s:s + 1], f"stream {s}: first page -> spare page {spare}")
    _others(ref, out, s, "spare first page")
    # and a repeat of the unplanted call is still green and bit-identical
    again = attend("decode", c, q)
    assert compare(again, ref)[0]
