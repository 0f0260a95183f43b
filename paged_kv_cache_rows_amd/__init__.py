"""Paged KV cache attention for MI355X (gfx950).

The compute path is the C-ABI library `libkvpaged.so` built from `csrc/` (hand-written HIP);
`paged_kv_cache_rows_amd.binding` loads it and wraps its entry points for torch tensors.
Importing this package alone loads nothing native.
"""
