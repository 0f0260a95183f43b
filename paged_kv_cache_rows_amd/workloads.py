"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle checks.

This module only draws inputs: shapes, per-stream lengths, page hand-out orders and
N(0, 1) values rounded to bf16.  It holds none of the attention arithmetic and none of the
page addressing, so both the HIP path and the float64 oracle can consume what it produces
without sharing any step of the method.

The shapes follow the workloads of TensorFold PR #1620 (paged K/V for Kolibri-1): pages of
512 positions, odd page sizes 37 and 64 from its kernel-contract bullet, 48/4 and 16/1 head
layouts at head dims 128 and 512 from the kernel-timing paragraph, 12 streams at a 40k
context from the maintainers' rerun, and the 1..8-row verify window of TensorFold PR #2730.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass
class Workload:
    """One synthetic layer call.

    lengths[s] is the stream's cache length after this call's rows are written; the call's
    `rows` rows sit at positions lengths[s] - rows .. lengths[s] - 1.
    """
    name: str
    streams: int
    kv_heads: int
    group: int
    head_dim: int
    page_size: int
    rows: int
    lengths: list
    window: int = 0
    ring_pages: int = 0
    spare_frac: float = 0.10
    min_spares: int = 0
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def q_heads(self) -> int:
        return self.kv_heads * self.group

    def pages_for(self, length: int) -> int:
        if self.ring_pages:
            return self.ring_pages
        return -(-length // self.page_size)

    @property
    def pages_used(self) -> int:
        return sum(self.pages_for(L) for L in self.lengths)

    @property
    def pool_pages(self) -> int:
        used = self.pages_used
        return max(used + self.min_spares, int(math.ceil(used * (1.0 + self.spare_frac))))

    @property
    def table_stride(self) -> int:
        return max(self.pages_for(L) for L in self.lengths)

    @property
    def kv_bytes_per_token(self) -> int:
        """K and V bytes of one position over all KV heads (bf16)."""
        return 2 * self.kv_heads * self.head_dim * 2


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def tiny_decode(seed: int = 1001) -> Workload:
    """1 stream, 1 KV head, GQA 4, d 128, 300 tokens in pages of 64 (5 used of an 8-page pool)."""
    return Workload("tiny_decode", streams=1, kv_heads=1, group=4, head_dim=128, page_size=64,
                    rows=1, lengths=[300], spare_frac=0.0, min_spares=3, seed=seed)


def batched_decode(seed: int = 1002, fixed_length: int | None = None) -> Workload:
    """12 streams, 8 KV heads, GQA 8, d 128, pages of 512, lengths uniform in [32768, 40960]."""
    if fixed_length is not None:
        lengths = [int(fixed_length)] * 12
        name = f"batched_decode_12x{fixed_length}"
    else:
        lengths = [int(x) for x in _rng(seed + 1000).integers(32768, 40960, size=12, endpoint=True)]
        name = "batched_decode"
    return Workload(name, streams=12, kv_heads=8, group=8, head_dim=128, page_size=512,
                    rows=1, lengths=lengths, spare_frac=0.10, seed=seed)


def verify_window(seed: int = 1003, rows: int = 8) -> Workload:
    """4 streams, 8 KV heads, GQA 8, d 128, pages of 512, about 9k tokens, 8 causal rows."""
    lengths = [int(x) for x in _rng(seed + 1000).integers(8800, 9200, size=4, endpoint=True)]
    return Workload("verify_window", streams=4, kv_heads=8, group=8, head_dim=128, page_size=512,
                    rows=rows, lengths=lengths, spare_frac=0.10, seed=seed)


def wide_head(seed: int = 1004) -> Workload:
    """2 streams, 2 KV heads, GQA 8, d 512, pages of 37; stream 0 decodes at 2048 (1 row),
    stream 1 verifies 4 rows at 9000.  Rows differ per stream, so the two streams are two
    calls on one pool; `rows` here is the verify call's and extra['rows'] lists both."""
    return Workload("wide_head", streams=2, kv_heads=2, group=8, head_dim=512, page_size=37,
                    rows=4, lengths=[2048, 9000], spare_frac=0.10, seed=seed,
                    extra={"rows": [1, 4]})


def prefill_mixed(seed: int = 1005, window: int = 0) -> Workload:
    """1 stream, a 2048-token prompt in 4 chunks of 512 rows, 8 KV heads, GQA 4, d 128, pages
    of 512.  window > 0 gives the sliding layer kept in a 3-page ring."""
    return Workload("prefill_window" if window else "prefill_full", streams=1, kv_heads=8,
                    group=4, head_dim=128, page_size=512, rows=512, lengths=[2048],
                    window=window, ring_pages=3 if window else 0, spare_frac=0.0,
                    min_spares=1, seed=seed, extra={"chunk": 512})


def free_order(num_pages: int, seed: int) -> np.ndarray:
    """A seeded permutation of the pool's page ids: the order pages are handed out."""
    return _rng(seed).permutation(num_pages).astype(np.int32)


def identity_order(num_pages: int) -> np.ndarray:
    return np.arange(num_pages, dtype=np.int32)


def normal_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """N(0, 1) draws in float32 from a seeded generator, rounded to bf16 (nearest even)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=dev)
    return x.to(torch.bfloat16)


def kv_history(w: Workload, device="cpu", salt: int = 0):
    """Per-stream K and V histories [L_s][Hkv][D] bf16 (the rows a stream has written)."""
    ks, vs = [], []
    for s, L in enumerate(w.lengths):
        ks.append(normal_bf16((L, w.kv_heads, w.head_dim), w.seed * 7919 + 2 * s + 1 + salt, device))
        vs.append(normal_bf16((L, w.kv_heads, w.head_dim), w.seed * 7919 + 2 * s + 2 + salt, device))
    return ks, vs


def queries(w: Workload, rows: int | None = None, device="cpu", salt: int = 0) -> torch.Tensor:
    """Queries [S][R][Hq][D] bf16."""
    R = w.rows if rows is None else rows
    return normal_bf16((w.streams, R, w.q_heads, w.head_dim), w.seed * 104729 + 17 + salt, device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw bf16 bit patterns of a tensor as uint16 numpy (a copy on the host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


# The canonical NaN pattern used to poison spare pages and unused slots, plus a second,
# negative signalling-looking pattern (both are NaN in bf16).
NAN_BITS = 0x7FC0
NAN_BITS_ALT = 0xFFC1


def all_workloads():
    return [tiny_decode(), batched_decode(), verify_window(), wide_head(), prefill_mixed()]
