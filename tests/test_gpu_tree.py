"""GPU parity tests of tree-shaped verify windows (paged_attn_verify_tree), through the C ABI.

Decode and drafted verify go through tree attention (TensorFold PR #1620, opening description,
Reads bullet): the drafts form a tree flattened into the window's slots, and each row sees the
keys before the window plus its own ancestors.  Both kernels are covered: VALU dots when rows
times the GQA group stay under 16, MFMA above.
"""
import numpy as np
import pytest
import torch

from gpu_support import assert_close, new_cache, oracle_tree_for, poisoned_workspace, random_tree_masks, say
from paged_kv_cache_rows_amd import binding, workloads

pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="tree", streams=3, kv_heads=2, group=8, head_dim=128, page_size=64, rows=8,
                lengths=[1500, 300, 8], spare_frac=0.2, min_spares=2, seed=31)
    base.update(kw)
    return workloads.Workload(**base)


def _tree(c, q, masks, window=0):
    m = torch.tensor(masks, dtype=torch.int32, device=c.table.device)
    ws = poisoned_workspace(c, q.shape[1], q.shape[2], window)
    out = binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, m, window=window, workspace=ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("G,R", [(4, 2), (4, 3), (8, 4), (8, 8), (4, 8), (8, 2)])
@pytest.mark.parametrize("P", [64, 37])
def test_random_trees_match_the_oracle(G, R, P):
    w = _w(group=G, rows=R, page_size=P, lengths=[1500, 300, R])
    say(f"tree G={G} R={R} P={P} ({'MFMA' if R * G >= 16 else 'VALU'})")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(R * 100 + G + P), w.streams, R)
    assert_close(_tree(c, q, masks), oracle_tree_for(c, q, masks), f"tree G={G} R={R} P={P}")


@pytest.mark.parametrize("G,R", [(4, 3), (8, 4), (8, 8)])
def test_random_trees_at_head_dim_512(G, R):
    # the d 512 kernels: VALU at 12 query vectors, MFMA at 32 (two waves without columns) and 64
    w = _w(group=G, rows=R, head_dim=512, kv_heads=1, page_size=37, lengths=[2000, 300, R])
    say(f"tree d512 G={G} R={R} ({'MFMA' if R * G >= 16 else 'VALU'})")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(R * 100 + G + 512), w.streams, R)
    assert_close(_tree(c, q, masks), oracle_tree_for(c, q, masks), f"tree d512 G={G} R={R}")


@pytest.mark.parametrize("G,R", [(4, 3), (8, 8)])
def test_chain_masks_equal_plain_verify_bytes(G, R):
    w = _w(group=G, rows=R)
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    chain = [[(1 << (r + 1)) - 1 for r in range(R)] for _ in range(w.streams)]
    plain = binding.verify(c.pool, q, c.table, c.seq_len, c.max_seq_len)
    torch.cuda.synchronize()
    assert torch.equal(_tree(c, q, chain).view(torch.int16), plain.view(torch.int16))


@pytest.mark.parametrize("G,R", [(4, 3), (8, 6)])
def test_tree_output_is_byte_equal_under_page_shuffles(G, R):
    w = _w(group=G, rows=R, lengths=[2100, 700, 90], page_size=64)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(7), w.streams, R)
    outs = []
    for kind in ("identity", 41, 42):
        c, _, _ = new_cache(w, identity=(kind == "identity"), order_seed=None if kind == "identity" else kind)
        outs.append(_tree(c, q, masks))
    for o in outs[1:]:
        assert torch.equal(outs[0].view(torch.int16), o.view(torch.int16))


@pytest.mark.parametrize("G,R,W", [(4, 3, 100), (8, 8, 300), (8, 8, 5)])
def test_trees_on_a_sliding_layer(G, R, W):
    w = _w(group=G, rows=R, window=W, lengths=[1200, 500, 64])
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(W), w.streams, R)
    assert_close(_tree(c, q, masks, window=W), oracle_tree_for(c, q, masks, window=W), f"tree window {W}")


def test_tree_verify_window_full_size():
    w = workloads.verify_window()
    say(f"tree verify window full size: lengths {w.lengths}")
    c, _, _ = new_cache(w)
    q = workloads.queries(w).cuda()
    masks = random_tree_masks(np.random.default_rng(99), w.streams, w.rows)
    assert_close(_tree(c, q, masks), oracle_tree_for(c, q, masks), "tree 4 streams x 8 rows")
