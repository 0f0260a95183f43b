"""Float64 CPU oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import anything here; the product path (the C-ABI library and its Python binding)
never does, and this package never imports the product path.

What it computes (TensorFold PR #1620, paged K/V for Kolibri-1's full layers):
  * `pages.gather_linear`   walks a stream's page table to rebuild its linear cache
                            (opening description, Reads bullet: keys are read through a
                            per-stream page table).
  * `pages.rows_put`        scatters a call's new K/V rows into their page slots
                            (opening description, Writes bullet).
  * `pages.copy_pages`      copies whole pages between ids (Kept states bullet: a stream's
                            state is kept by copying the pages its table walks).
  * `attention.attend`      softmax(q k^T / sqrt(d)) v over the linear cache, with GQA, causal
                            verify rows and an optional sliding window, all in float64 (the
                            author's kernel-timing reply: the paged kernels read the same
                            keys as the linear ones, so the result is the linear cache's).
  * `attention.attend_stream_tree`
                            the same over a tree-shaped verify window: every key before the
                            window plus the row's ancestor slots (decode and drafted verify go
                            through tree attention in the opening description's Reads bullet).
  * `lease.LeaseModel`      the pool's page hand-out and return, as a plain Python model
                            (opening description: every stream leases pages as it grows).

Pins: every function above is pinned by tests that do not reuse its code (brute force in
pure Python, closed forms, permutation invariance, a library special case, invariants);
see the module docstrings for which pin covers what.
"""
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits
from .attention import (attend, attend_stream, attend_stream_tree, tree_keys, visible_range, row_position,
                        kv_head_of)
from .pages import copy_pages, gather_linear, rows_put, slot_of
from .lease import LeaseModel, NoPages

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "attend", "attend_stream", "attend_stream_tree", "tree_keys",
    "visible_range",
    "row_position", "kv_head_of", "copy_pages", "gather_linear", "rows_put", "slot_of", "LeaseModel",
    "NoPages",
]
