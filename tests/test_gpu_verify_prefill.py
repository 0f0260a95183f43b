"""GPU parity tests of the MFMA path (rows x GQA group >= 16): speculative verify windows of
2..8 causal rows (TensorFold PR #2730) and prompt chunks (TensorFold PR #1620, prompt kernels
over pages), including the sliding-window layer kept in a ring, through the C ABI.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_support import (assert_close, attend, new_cache, oracle_for, oracle_from_history, pool_bits,
                         remember, say)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="t", streams=2, kv_heads=2, group=8, head_dim=128, page_size=64, rows=8,
                lengths=[700, 97], spare_frac=0.2, min_spares=2, seed=9)
    base.update(kw)
    return workloads.Workload(**base)


# ----------------------------------------------------------------------------- verify windows
def test_verify_window_full_size_all_streams():
    w = workloads.verify_window()
    say(f"verify window: lengths {w.lengths}, rows {w.rows}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q)
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q), "verify 4 streams x 8 rows")


@pytest.mark.parametrize("G,R", [(8, 2), (8, 3), (8, 5), (8, 8), (4, 4), (4, 6), (4, 8)])
@pytest.mark.parametrize("P", [64, 37, 512])
def test_verify_rows_parity(G, R, P):
    w = _w(group=G, rows=R, page_size=P, lengths=[1500, 300, R], streams=3)
    say(f"verify G={G} R={R} P={P}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q), oracle_for(c, q), f"verify G={G} R={R} P={P}")


@pytest.mark.parametrize("L", [2000, 5000, 6100, 7000, 13000])
@pytest.mark.parametrize("P", [64, 37])
def test_verify_splits_of_many_step_counts(L, P):
    # 4 streams x 8 KV heads: the plan cuts each stream into 8 chunks of about L / 8 keys, so a
    # split runs 2, 5, 6, 7 or 13 two-tile steps: the pipeline's main loop, its tail without
    # loads past the split, and the boundary between them; shorter streams end mid-chunk
    w = _w(streams=4, kv_heads=8, group=8, rows=8, page_size=P, lengths=[L, L - 37, L // 2, 9])
    say(f"verify splits L={L} P={P}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q), oracle_for(c, q), f"verify L={L} P={P}")


@pytest.mark.parametrize("L", [2300, 2700, 3100, 3600, 4100])
@pytest.mark.parametrize("P", [64, 512])
@pytest.mark.parametrize("W", [0, 77])
def test_verify_split_pipeline_depths(L, P, W):
    # pages a multiple of 64 keys: the split calls' kernel with 32-key sub-tiles in four buffers
    # per operand.  Chunks of about L / 8 keys give 5 to 9 steps of 64 keys, where its loads
    # stay in flight across barriers only while four more groups of them have been issued in
    # full; a window of 77 starts each row's keys off a sub-tile boundary
    w = _w(streams=4, kv_heads=8, group=8, rows=8, page_size=P, lengths=[L, L - 45, L // 2 + 3, 9])
    say(f"verify split pipeline L={L} P={P} W={W}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q, window=W), oracle_for(c, q, W), f"verify L={L} P={P} W={W}")


@pytest.mark.parametrize("entry,R,G,D,Hkv", [("decode", 1, 8, 128, 2), ("verify", 3, 4, 128, 2),
                                              ("verify", 8, 8, 128, 2), ("verify", 4, 8, 512, 1),
                                              ("prefill", 100, 4, 128, 2), ("prefill", 512, 4, 128, 8)])
def test_rows_before_the_stream_are_zeros(entry, R, G, D, Hkv):
    # a stream of length 0 and one shorter than the call's rows: rows at negative positions see
    # no key and come out as zeros on every path (VALU, MFMA split, MFMA direct for 512 rows),
    # the other rows as the oracle's; the NaN workspace must not leak into them
    lengths = [700, 0, max(1, R - 3)]
    w = _w(group=G, rows=R, head_dim=D, kv_heads=Hkv, page_size=64, lengths=lengths, streams=3)
    say(f"rows before the stream: {entry} R={R} G={G} D={D}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend(entry, c, q)
    assert torch.isfinite(out.float()).all()
    assert (out[1].view(torch.int16) == 0).all()
    assert (out[2, :R - lengths[2]].view(torch.int16) == 0).all()
    assert_close(out, oracle_for(c, q), f"{entry} R={R} with short streams")


@pytest.mark.parametrize("entry,R,G,D", [("decode", 1, 8, 128), ("verify", 2, 4, 128), ("verify", 8, 8, 128),
                                         ("verify", 4, 8, 512), ("prefill", 64, 4, 128)])
def test_peaked_softmax_with_a_late_dominant_key(entry, R, G, D):
    # K and q scaled by 6 (scores about 36 times larger), and one key near the end of stream 0
    # set along its first query head: that row's weights are close to one-hot and the running
    # max jumps late, after many tiles, which exercises the rescale of every path
    w = _w(group=G, rows=R, head_dim=D, kv_heads=2 if D == 128 else 1, page_size=64,
           lengths=[2300, 900], streams=2)
    say(f"peaked softmax: {entry} R={R} G={G} D={D}")
    c, _, _ = new_cache(w, history=False)
    ks, vs = workloads.kv_history(w)
    q = (workloads.queries(w).float() * 6).to(torch.bfloat16)
    ks = [(k.float() * 6).to(torch.bfloat16) for k in ks]
    p = c.lengths[0] - R - 40
    ks[0][p, 0] = (q[0, 0, 0].float() * 2).to(torch.bfloat16)
    staging.write_history(c, ks, vs)
    remember(c, ks, vs)
    q = q.cuda()
    out = attend(entry, c, q)
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q), f"peaked {entry} R={R} D={D}")


@pytest.mark.parametrize("entry,R,G,D", [("decode", 1, 8, 128), ("decode", 1, 4, 512), ("verify", 3, 4, 128),
                                         ("verify", 8, 8, 128), ("verify", 4, 8, 512), ("prefill", 64, 4, 128),
                                         ("prefill", 512, 4, 128)])
@pytest.mark.parametrize("scale", [0.02, 0.25])
def test_explicit_scale_on_every_path(entry, R, G, D, scale):
    # a caller-given scale in place of 1/sqrt(d) (0.088 at d 128, 0.044 at d 512): flatter and
    # sharper weights on the VALU path, the MFMA split at d 128 and 512 and the direct plan
    Hkv = 8 if R == 512 else (2 if D == 128 else 1)
    w = _w(group=G, rows=R, head_dim=D, kv_heads=Hkv, page_size=64, lengths=[1500, 600], streams=2)
    say(f"scale {scale}: {entry} R={R} G={G} D={D}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend(entry, c, q, scale=scale)
    assert torch.isfinite(out.float()).all()
    assert_close(out, oracle_for(c, q, scale=scale), f"{entry} R={R} D={D} scale {scale}")
    # the scale reaches the kernels: the default gives different bytes
    assert not torch.equal(out.view(torch.int16), attend(entry, c, q).view(torch.int16))


def test_verify_is_byte_equal_under_shuffles_and_repeat():
    w = _w(lengths=[2500, 1300, 800], streams=3, page_size=512)
    q = workloads.queries(w).cuda()
    outs = []
    for kind in ("identity", 21, 22):
        c, _, _ = new_cache(w, identity=(kind == "identity"), order_seed=None if kind == "identity" else kind)
        outs.append(attend("verify", c, q))
    outs.append(attend("verify", c, q))
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))
    assert_close(outs[0], oracle_for(c, q), "verify shuffled")


def test_verify_rows_match_decode_at_their_lengths():
    w = _w(lengths=[1800, 900], rows=8)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    out = attend("verify", c, q)
    for r in range(8):
        lens = [L - 8 + r + 1 for L in c.lengths]
        seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
        one = binding.decode(c.pool, q[:, r:r + 1].contiguous(), c.table, seq, c.max_seq_len)
        torch.cuda.synchronize()
        ref = oracle_for(c, q[:, r:r + 1].contiguous(), lengths=lens)
        assert_close(one, ref, f"row {r} via decode")
        assert_close(out[:, r:r + 1], ref, f"row {r} via verify")


@pytest.mark.parametrize("W", [1, 7, 300])
def test_verify_sliding_window(W):
    w = _w(lengths=[1500, 400], window=W)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q, window=W), oracle_for(c, q, window=W), f"verify window {W}")


# ----------------------------------------------------------------------------- wide head
def test_wide_head_pair_with_nan_in_unused_slots():
    w = workloads.wide_head()
    assert w.page_size == 37 and w.head_dim == 512
    c, ks, vs = new_cache(w)
    kb, vb = pool_bits(c)
    # the last page of each stream has unused slots, and they hold the NaN pattern
    for s, L in enumerate(c.lengths):
        last = c.table_host[s][(L - 1) // 37]
        used = L - ((L - 1) // 37) * 37
        if used < 37:
            assert (kb[last, :, used:] == workloads.NAN_BITS).all()
    # stream 0: one decode row at 2048 (VALU); stream 1: four verify rows at 9000 (MFMA)
    q0 = workloads.normal_bf16((1, 1, w.q_heads, 512), 4101).cuda()
    q1 = workloads.normal_bf16((1, 4, w.q_heads, 512), 4102).cuda()
    t0, l0 = c.stream_view(0)
    t1, l1 = c.stream_view(1)
    o0 = binding.decode(c.pool, q0, t0, l0, c.lengths[0])
    o1 = binding.verify(c.pool, q1, t1, l1, c.lengths[1])
    torch.cuda.synchronize()
    assert_close(o0, oracle_from_history(ks[:1], vs[:1], q0, c.lengths[:1]), "wide decode L=2048")
    assert_close(o1, oracle_from_history(ks[1:], vs[1:], q1, c.lengths[1:]), "wide verify L=9000 R=4")


# ----------------------------------------------------------------------------- prefill
def _prefill_chunks(w, window=0):
    """Write a 2048-token prompt chunk by chunk and attend each chunk; returns the per-chunk
    outputs, the oracle's and the history."""
    c, _, _ = new_cache(w, history=False, lengths=[2048])
    ks, vs = workloads.kv_history(w)
    q_all = workloads.normal_bf16((1, 2048, w.q_heads, w.head_dim), w.seed * 31 + 5)
    outs, refs = [], []
    for c0 in range(0, 2048, 512):
        c1 = c0 + 512
        seq = torch.tensor([c1], dtype=torch.int32, device="cuda")
        binding.rows_put(c.pool, c.table, seq, ks[0][c0:c1].cuda()[None].contiguous(),
                         vs[0][c0:c1].cuda()[None].contiguous(), max_seq_len=c1, ring_pages=c.ring_pages)
        q = q_all[:, c0:c1].contiguous().cuda()
        out = binding.prefill(c.pool, q, c.table, seq, 2048, window=window, ring_pages=c.ring_pages)
        torch.cuda.synchronize()
        outs.append(out)
        refs.append(oracle_from_history(ks, vs, q, [c1], window))
    return c, outs, refs


def test_prefill_full_layer_in_512_row_chunks():
    w = workloads.prefill_mixed()
    say(f"prefill full: {w.q_heads} q heads / {w.kv_heads} kv heads, P {w.page_size}")
    c, outs, refs = _prefill_chunks(w)
    for i, (o, r) in enumerate(zip(outs, refs)):
        assert torch.isfinite(o.float()).all()
        assert_close(o, r, f"full layer chunk {i}")


def test_prefill_sliding_layer_on_a_ring():
    w = workloads.prefill_mixed(window=1024)
    assert w.ring_pages == 3 and w.window == 1024
    c, outs, refs = _prefill_chunks(w, window=1024)
    for i, (o, r) in enumerate(zip(outs, refs)):
        assert_close(o, r, f"window layer chunk {i}")


def test_prefill_chunked_equals_one_call():
    w = _w(group=4, rows=256, lengths=[1024], streams=1, kv_heads=2, page_size=64)
    c, ks, vs = new_cache(w)
    q = workloads.normal_bf16((1, 1024, w.q_heads, 128), 77).cuda()
    whole = binding.prefill(c.pool, q, c.table, c.seq_len, 1024)
    parts = []
    for c0 in range(0, 1024, 256):
        seq = torch.tensor([c0 + 256], dtype=torch.int32, device="cuda")
        parts.append(binding.prefill(c.pool, q[:, c0:c0 + 256].contiguous(), c.table, seq, 1024))
    torch.cuda.synchronize()
    ref = oracle_from_history(ks, vs, q, [1024])
    assert_close(whole, ref, "prefill one call")
    assert_close(torch.cat(parts, dim=1), ref, "prefill in chunks")


@pytest.mark.parametrize("R", [1, 3, 17, 100])
def test_prefill_small_and_ragged_row_counts(R):
    w = _w(group=4, rows=R, lengths=[R, R + 500], streams=2, page_size=37)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("prefill", c, q), oracle_for(c, q), f"prefill R={R}")


@pytest.mark.parametrize("D", [128, 512])
def test_prefill_wide_and_narrow_heads_with_window(D):
    w = _w(group=8, rows=40, head_dim=D, kv_heads=1, lengths=[600], streams=1, page_size=37, window=70)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("prefill", c, q, window=70), oracle_for(c, q, window=70), f"prefill D={D} W=70")
