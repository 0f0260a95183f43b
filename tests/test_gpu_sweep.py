"""A seeded random sweep of call shapes against the oracle, through the C ABI.

Each case draws an entry point (decode, decode with the fused row write, verify, tree verify,
prompt chunk), head dim, GQA group, rows, page size, KV heads, stream count and ragged lengths,
and a full or sliding-window layer (sometimes kept in a ring of pages), so that combinations
the targeted tests do not list are covered too.  The cases are fixed by the seed; each prints
its shape before it runs.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_support import (assert_close, new_cache, oracle_for, oracle_from_history, oracle_tree_for,
                         poisoned_workspace, random_tree_masks, say)
from paged_kv_cache_rows_amd import binding, staging, workloads

pytestmark = pytest.mark.gpu

SEED = 5150
N_CASES = 48


@dataclasses.dataclass
class Case:
    entry: str
    D: int
    G: int
    R: int
    P: int
    Hkv: int
    lengths: list
    window: int
    ring: int

    def __str__(self):
        return (f"{self.entry} D{self.D} G{self.G} R{self.R} P{self.P} Hkv{self.Hkv} L{self.lengths} "
                f"W{self.window} ring{self.ring}")


def _cases():
    rng = np.random.default_rng(SEED)
    out = []
    while len(out) < N_CASES:
        entry = ["decode", "decode_put", "verify", "tree", "prefill"][int(rng.integers(0, 5))]
        D = int(rng.choice([128, 512]))
        G = int(rng.choice([4, 8, 12, 16]))
        R = {"decode": 1, "decode_put": 1, "verify": int(rng.integers(1, 9)),
             "tree": int(rng.integers(2, 9)), "prefill": int(rng.integers(9, 129))}[entry]
        P = int(rng.choice([1, 3, 16, 37, 64, 100, 512]))
        Hkv = 1 if D == 512 or G >= 12 else int(rng.integers(1, 3))
        S = int(rng.integers(1, 5))
        top = 6000 if D == 128 else 3000
        if P == 1:
            top = 1500
        lengths = [int(rng.integers(max(R, 1), top + 1)) for _ in range(S)]
        window = 0
        ring = 0
        if rng.random() < 0.4:
            window = int(rng.integers(1, 2500))
            if rng.random() < 0.5:
                ring = -(-(window + R - 1) // P) + int(rng.integers(0, 3))
                if ring > 2000:
                    ring = 0
        out.append(Case(entry, D, G, R, P, Hkv, lengths, window, ring))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_random_shape_matches_the_oracle(case):
    say(f"sweep {case}")
    w = workloads.Workload(name="sweep", streams=len(case.lengths), kv_heads=case.Hkv, group=case.G,
                           head_dim=case.D, page_size=case.P, rows=case.R, lengths=case.lengths,
                           window=case.window, ring_pages=case.ring, spare_frac=0.15, min_spares=2,
                           seed=SEED + CASES.index(case))
    q = workloads.queries(w).cuda()
    W = case.window
    if case.entry == "decode_put":
        ks, vs = workloads.kv_history(w)
        c = staging.make_cache(w, order=workloads.free_order(w.pool_pages, w.seed + 1))
        staging.write_history(c, ks, vs, upto=[L - 1 for L in case.lengths])
        dev = c.table.device
        k_new = torch.stack([ks[s][L - 1:L] for s, L in enumerate(case.lengths)]).to(dev).contiguous()
        v_new = torch.stack([vs[s][L - 1:L] for s, L in enumerate(case.lengths)]).to(dev).contiguous()
        out = binding.decode_put(c.pool, q, c.table, c.seq_len, c.max_seq_len, k_new, v_new, window=W,
                                 ring_pages=c.ring_pages, workspace=poisoned_workspace(c, 1, w.q_heads, W))
        torch.cuda.synchronize()
        ref = oracle_from_history(ks, vs, q, case.lengths, W)
    else:
        c, _, _ = new_cache(w)
        ws = poisoned_workspace(c, case.R, w.q_heads, W)
        if case.entry == "tree":
            masks = random_tree_masks(np.random.default_rng(w.seed), w.streams, case.R)
            m = torch.tensor(masks, dtype=torch.int32, device=c.table.device)
            out = binding.verify_tree(c.pool, q, c.table, c.seq_len, c.max_seq_len, m, window=W,
                                      ring_pages=c.ring_pages, workspace=ws)
            torch.cuda.synchronize()
            ref = oracle_tree_for(c, q, masks, W)
        else:
            fn = {"decode": binding.decode, "verify": binding.verify, "prefill": binding.prefill}[case.entry]
            out = fn(c.pool, q, c.table, c.seq_len, c.max_seq_len, window=W, ring_pages=c.ring_pages,
                     workspace=ws)
            torch.cuda.synchronize()
            ref = oracle_for(c, q, W)
    assert_close(out, ref, str(case))


def test_the_sweep_spans_both_kernels_and_every_entry():
    kinds = {(c.entry, "MFMA" if c.R * c.G >= 16 else "VALU") for c in CASES}
    assert {e for e, _ in kinds} == {"decode", "decode_put", "verify", "tree", "prefill"}
    assert {k for _, k in kinds} == {"MFMA", "VALU"}
    assert any(c.ring for c in CASES) and any(c.window and not c.ring for c in CASES)
    assert {c.D for c in CASES} == {128, 512} and {c.G for c in CASES} == {4, 8, 12, 16}
