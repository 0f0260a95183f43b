"""GPU parity tests of the channel-split kernel at head dim 512 (16 to 32 query vectors per KV
head over pages of at least 32 keys), through the C ABI.

These are the head-dim-512 layer's verify rows (TensorFold PR #1620, per-tile follow-up) when a
window holds a few rows. Each of the kernel's four waves takes a quarter of the channels, and the
waves' partial scores are added in LDS. Covered here:
  - one and two 16-column query blocks;
  - pages that are a multiple of the 32-key tile, and pages that straddle tiles;
  - chunks of one or several 3-tile batches, and last batches of one or two tiles;
  - windows over a full table and over a ring, and draft trees;
  - NaN in unused slots and in the workspace;
  - byte equality under another page order and under the identity table;
  - controls that must go red.
"""
import numpy as np
import pytest
import torch

from gpu_support import (assert_close, assert_red, attend, new_cache, oracle_for, oracle_from_history,
                         oracle_tree_for, poisoned_workspace, random_tree_masks, say)
from paged_kv_cache_rows_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _w(G, R, P, lengths, Hkv=1, seed=171, **kw):
    return workloads.Workload(name="narrow", streams=len(lengths), kv_heads=Hkv, group=G, head_dim=512,
                              page_size=P, rows=R, lengths=lengths, spare_frac=0.1, min_spares=2, seed=seed, **kw)


def _entry(R):
    return "decode" if R == 1 else "verify"


# query vectors R * G: 16 (one block) or 24 and 32 (two); pages of 32, 37, 64, 100 and 512;
# lengths whose chunks end on every tile of a batch
@pytest.mark.parametrize("G,R", [(8, 2), (8, 4), (4, 4), (4, 8), (12, 2), (16, 1), (16, 2)])
@pytest.mark.parametrize("P", [37, 64, 512])
def test_channel_split_parity(G, R, P):
    w = _w(G, R, P, [2000, 97, 129, 33, R], Hkv=2, seed=171 + P + 10 * G + R)
    say(f"channel-split d512 G={G} R={R} P={P}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend(_entry(R), c, q), oracle_for(c, q), f"G={G} R={R} P={P}")


@pytest.mark.parametrize("P", [32, 100])
def test_channel_split_page_sizes(P):
    w = _w(8, 4, P, [3001, 500, 31], Hkv=2, seed=181 + P)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q), oracle_for(c, q), f"P={P}")


@pytest.mark.parametrize("L,P", [(20000, 37), (40000, 512), (40001, 64)])
def test_channel_split_several_batches_per_chunk(L, P):
    # 2 KV heads at 20k-40k keys: more chunks of 96 keys than one round of 256 workgroups holds,
    # so the plan gives chunks of 2 to 4 batches of 3 tiles
    w = _w(8, 4, P, [L], Hkv=2, seed=191)
    say(f"channel-split d512 L={L} P={P}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q), oracle_for(c, q), f"L={L} P={P}")


def test_channel_split_bytes_under_page_order_and_identity_table():
    w = _w(8, 4, 37, [9000, 1000, 40], Hkv=2, seed=201)
    outs = []
    for kw in (dict(), dict(order_seed=7), dict(identity=True)):
        c, _, _ = new_cache(w, **kw)
        q = workloads.queries(w).cuda()
        outs.append(attend("verify", c, q).cpu())
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


@pytest.mark.parametrize("W", [1, 40, 300, 5000])
def test_channel_split_window(W):
    w = _w(8, 4, 37, [9000, 700, 4], Hkv=2, seed=211)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q, window=W), oracle_for(c, q, window=W), f"window {W}")


def test_channel_split_ring_layer():
    W, P, ring = 100, 64, 2            # ring of 128 positions holds window + rows - 1
    w = _w(8, 4, P, [1000, 300], Hkv=2, window=W, ring_pages=ring, seed=221)
    c, ks, vs = new_cache(w)
    q = workloads.queries(w).cuda()
    assert_close(attend("verify", c, q, window=W), oracle_from_history(ks, vs, q, c.lengths, W), "ring")


@pytest.mark.parametrize("G,R,P", [(8, 4, 64), (4, 8, 37), (8, 2, 512)])
def test_channel_split_trees(G, R, P):
    w = _w(G, R, P, [2000, 300, R], Hkv=2, seed=231)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(G * 100 + R + P), w.streams, R)
    m = torch.tensor(masks, dtype=torch.int32, device=c.table.device)
    ws = poisoned_workspace(c, q.shape[1], q.shape[2])
    out = binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, m, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out, oracle_tree_for(c, q, masks), f"tree G={G} R={R} P={P}")


def test_channel_split_controls_go_red():
    # the wide-head verify (4 rows x GQA 8 at 9,000 keys over pages of 37): query heads permuted
    # inside each KV group, a stream one key short, one table entry on another page of the stream
    # (a duplicate: swapping two fully visible pages would only reorder the keys, which attention
    # does not see)
    w = _w(8, 4, 37, [9000], Hkv=2, seed=241)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    ref = oracle_for(c, q)
    assert_close(attend("verify", c, q), ref, "clean")
    perm = torch.arange(w.q_heads).view(w.kv_heads, w.group).flip(1).reshape(-1)
    assert_red(attend("verify", c, q[:, :, perm].contiguous()), ref, "query heads permuted")
    c.seq_len -= 1
    assert_red(attend("verify", c, q), ref, "length one short")
    c.seq_len += 1
    t0 = c.table.clone()
    c.table[0, 3] = t0[0, 7].item()
    assert_red(attend("verify", c, q), ref, "one table entry on another page of the stream")
    c.table.copy_(t0)
    assert_close(attend("verify", c, q), ref, "clean again")
