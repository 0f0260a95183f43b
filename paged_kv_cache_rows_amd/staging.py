"""Build a paged cache for a workload through the library's own entry points.

Creates the pool (pages pre-filled with a NaN pattern), leases each stream's pages in stream
order through kv_page_lease (so a shuffled free order gives shuffled tables and the identity
order gives contiguous, "linear" tables), uploads the page table, and writes each stream's
history with kv_rows_put in chunks.  Nothing here computes attention.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import binding
from .workloads import NAN_BITS, Workload


@dataclass
class Cache:
    w: Workload
    pool: binding.Pool
    table: torch.Tensor          # device int32 [S][stride]
    table_host: np.ndarray       # the same on the host
    seq_len: torch.Tensor        # device int32 [S]
    lengths: list
    max_seq_len: int
    ring_pages: int

    def stream_view(self, s: int):
        """(table, seq_len) views of one stream, for per-stream calls."""
        return self.table[s:s + 1], self.seq_len[s:s + 1]


def make_cache(w: Workload, device="cuda", order=None, fill_bits: int = NAN_BITS,
               lengths=None, lease_policy: int | None = None, grow_in_turn: int = 0) -> Cache:
    """`lease_policy`: set on the pool before any lease (KV_LEASE_QUEUE by default).
    `grow_in_turn` > 0: the streams lease their pages in turns of that many pages each, as
    streams that grow side by side do; 0: each stream leases all its pages at once."""
    lengths = list(w.lengths if lengths is None else lengths)
    pool = binding.Pool(w.pool_pages, w.page_size, w.kv_heads, w.head_dim, max_streams=w.streams,
                        device=device, free_order=order, fill_bits=fill_bits)
    if lease_policy is not None:
        pool.set_lease_policy(lease_policy)
    stride = w.table_stride
    table = np.full((w.streams, stride), -1, dtype=np.int32)
    need = [w.pages_for(L) for L in lengths]
    have = [0] * len(lengths)
    turn = grow_in_turn if grow_in_turn > 0 else max(need + [1])
    while any(h < n for h, n in zip(have, need)):
        for s in range(len(lengths)):
            k = min(turn, need[s] - have[s])
            if k > 0:
                ids = pool.lease(s, k)
                table[s, have[s]:have[s] + k] = ids
                have[s] += k
    table_d = torch.from_numpy(table).to(device)
    seq = torch.tensor(lengths, dtype=torch.int32, device=device)
    return Cache(w, pool, table_d, table, seq, lengths, max(lengths), w.ring_pages)


def write_history(c: Cache, ks, vs, upto=None, chunk_rows: int = 4096):
    """Write rows [0, upto[s]) of each stream's history (default: all of it) with kv_rows_put,
    chunk by chunk in position order."""
    dev = c.table.device
    for s in range(c.w.streams):
        L = c.lengths[s] if upto is None else upto[s]
        t, _ = c.stream_view(s)
        step = chunk_rows
        if c.ring_pages:
            step = min(step, c.ring_pages * c.w.page_size)
        for c0 in range(0, L, step):
            c1 = min(L, c0 + step)
            seq = torch.tensor([c1], dtype=torch.int32, device=dev)
            kn = ks[s][c0:c1].to(dev).unsqueeze(0).contiguous()
            vn = vs[s][c0:c1].to(dev).unsqueeze(0).contiguous()
            binding.rows_put(c.pool, t, seq, kn, vn, max_seq_len=c1, ring_pages=c.ring_pages)
