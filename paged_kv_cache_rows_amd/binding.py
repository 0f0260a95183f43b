"""Python binding of libkvpaged.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module checks dtypes, devices
and shapes of torch tensors, fills the C structs of include/kvpaged.h and passes
torch.cuda.current_stream() as the HIP stream.  There is no fallback: if the library is
missing or fails to load, every call raises.

torch is imported before the library is loaded so that both use the one HIP runtime
(torch's libamdhip64.so.7 satisfies the library's dependency of the same soname).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_size_t, c_void_p

import numpy as np
import torch

# KVPAGED_LIB names another build of the library (the host sanitizer tests load one)
LIB_PATH = os.environ.get("KVPAGED_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvpaged.so")

KV_OK, KV_E_ARG, KV_E_SHAPE, KV_E_NO_PAGES, KV_E_WORKSPACE, KV_E_DEVICE = 0, -1, -2, -3, -4, -5
KV_LEASE_QUEUE, KV_LEASE_CONTIGUOUS = 0, 1
STATUS_NAMES = {0: "KV_OK", -1: "KV_E_ARG", -2: "KV_E_SHAPE", -3: "KV_E_NO_PAGES",
                -4: "KV_E_WORKSPACE", -5: "KV_E_DEVICE"}

# The entry points include/kvpaged.h declares (checked against the built library's exports).
EXPORTS = ("kv_pool_create", "kv_pool_destroy", "kv_page_lease", "kv_page_release", "kv_page_share",
           "kv_pool_set_lease_policy",
           "kv_pool_free_count", "kv_stream_pages", "kv_rows_put", "kv_pages_copy", "paged_attn_workspace_size",
           "paged_attn_decode", "paged_attn_decode_put", "paged_attn_decode_put_static", "paged_attn_verify", "paged_attn_verify_tree",
           "paged_attn_prefill", "paged_attn_prefill_put",
           "kv_set_part_events",
           "kv_last_error", "kv_abi_version")


class KvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_pages", c_int32), ("page_size", c_int32), ("num_kv_heads", c_int32),
                ("head_dim", c_int32), ("max_streams", c_int32), ("k_pages", c_void_p),
                ("v_pages", c_void_p), ("free_order", POINTER(c_int32))]


class Layout(ctypes.Structure):
    _fields_ = [("num_streams", c_int32), ("rows", c_int32), ("page_table", c_void_p),
                ("table_stride", c_int32), ("seq_len", c_void_p), ("max_seq_len", c_int32),
                ("ring_pages", c_int32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("q", c_void_p), ("out", c_void_p), ("num_q_heads", c_int32), ("scale", c_float),
                ("window", c_int32), ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_rows_amd.build`")
    lib = ctypes.CDLL(path)
    i32p = POINTER(c_int32)
    sig = {
        "kv_pool_create": [POINTER(PoolDesc), POINTER(c_void_p)],
        "kv_pool_destroy": [c_void_p],
        "kv_page_lease": [c_void_p, c_int32, c_int32, i32p],
        "kv_page_release": [c_void_p, c_int32],
        "kv_page_share": [c_void_p, c_int32, c_int32, c_int32],
        "kv_pool_set_lease_policy": [c_void_p, c_int32],
        "kv_pool_free_count": [c_void_p, i32p],
        "kv_stream_pages": [c_void_p, c_int32, i32p, c_int32, i32p],
        "kv_rows_put": [c_void_p, POINTER(Layout), c_void_p, c_void_p, c_void_p],
        "kv_pages_copy": [c_void_p, c_void_p, c_void_p, c_int32, c_void_p],
        "paged_attn_workspace_size": [c_void_p, POINTER(Layout), POINTER(AttnArgs), POINTER(c_size_t)],
        "paged_attn_decode": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p],
        "paged_attn_decode_put": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p, c_void_p, c_void_p],
        "paged_attn_decode_put_static": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p, c_void_p,
                                         c_void_p],
        "paged_attn_verify": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p],
        "paged_attn_verify_tree": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p, c_void_p],
        "paged_attn_prefill": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p],
        "paged_attn_prefill_put": [c_void_p, POINTER(Layout), POINTER(AttnArgs), c_void_p, c_void_p, c_void_p],
        "kv_set_part_events": [c_void_p, c_void_p],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int32
    lib.kv_last_error.argtypes = []
    lib.kv_last_error.restype = ctypes.c_char_p
    lib.kv_abi_version.argtypes = []
    lib.kv_abi_version.restype = c_int32
    _lib = lib
    return lib


def _check(status: int):
    if status != KV_OK:
        raise KvError(status, load().kv_last_error().decode(errors="replace"))


def _stream_handle(stream=None) -> int:
    if not torch.cuda.is_available():
        return 0
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class Pool:
    """A page pool: caller-side K/V page tensors [num_pages][Hkv][P][D] bf16 plus the
    library's lease bookkeeping.  New pages are filled with `fill_bits` (a NaN pattern by
    default), so that any read of a slot that was never written shows up."""

    def __init__(self, num_pages: int, page_size: int, kv_heads: int, head_dim: int,
                 max_streams: int, device="cuda", free_order=None, fill_bits: int | None = 0x7FC0,
                 k_pages: torch.Tensor | None = None, v_pages: torch.Tensor | None = None):
        lib = load()
        shape = (num_pages, kv_heads, page_size, head_dim)
        if k_pages is None:
            k_pages = torch.empty(shape, dtype=torch.bfloat16, device=device)
            v_pages = torch.empty(shape, dtype=torch.bfloat16, device=device)
            if fill_bits is not None:
                fb = int(np.array([fill_bits], dtype=np.uint16).view(np.int16)[0])
                k_pages.view(torch.int16).fill_(fb)
                v_pages.view(torch.int16).fill_(fb)
        _need(k_pages, torch.bfloat16, "k_pages", shape)
        _need(v_pages, torch.bfloat16, "v_pages", shape)
        self.k_pages, self.v_pages = k_pages, v_pages
        self.num_pages, self.page_size = num_pages, page_size
        self.kv_heads, self.head_dim, self.max_streams = kv_heads, head_dim, max_streams
        self._order = None
        fo = None
        if free_order is not None:
            self._order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            fo = self._order.ctypes.data_as(POINTER(c_int32))
        desc = PoolDesc(num_pages, page_size, kv_heads, head_dim, max_streams,
                        _ptr(k_pages), _ptr(v_pages), fo)
        h = c_void_p()
        _check(lib.kv_pool_create(ctypes.byref(desc), ctypes.byref(h)))
        self.handle = h

    def lease(self, stream: int, n: int) -> list:
        ids = (c_int32 * max(n, 1))()
        _check(load().kv_page_lease(self.handle, stream, n, ids))
        return [int(ids[i]) for i in range(n)]

    def set_lease_policy(self, policy: int):
        """KV_LEASE_QUEUE (default) or KV_LEASE_CONTIGUOUS: which free ids later leases take."""
        _check(load().kv_pool_set_lease_policy(self.handle, policy))

    def release(self, stream: int):
        _check(load().kv_page_release(self.handle, stream))

    def share(self, src_stream: int, dst_stream: int, n: int):
        """kv_page_share: dst_stream (holding no pages) takes src_stream's first n pages."""
        _check(load().kv_page_share(self.handle, src_stream, dst_stream, n))

    def free_count(self) -> int:
        n = c_int32()
        _check(load().kv_pool_free_count(self.handle, ctypes.byref(n)))
        return int(n.value)

    def stream_pages(self, stream: int) -> list:
        n = c_int32()
        _check(load().kv_stream_pages(self.handle, stream, None, 0, ctypes.byref(n)))
        ids = (c_int32 * max(n.value, 1))()
        _check(load().kv_stream_pages(self.handle, stream, ids, n.value, ctypes.byref(n)))
        return [int(ids[i]) for i in range(n.value)]

    def close(self):
        if getattr(self, "handle", None):
            load().kv_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _layout(pool: Pool, table: torch.Tensor, seq_len: torch.Tensor, rows: int, max_seq_len: int,
            ring_pages: int) -> Layout:
    _need(table, torch.int32, "page_table")
    _need(seq_len, torch.int32, "seq_len")
    if table.dim() != 2 or seq_len.dim() != 1 or table.shape[0] != seq_len.shape[0]:
        raise ValueError("page_table must be [S][stride] and seq_len [S]")
    return Layout(int(seq_len.shape[0]), int(rows), _ptr(table), int(table.shape[1]), _ptr(seq_len),
                  int(max_seq_len), int(ring_pages))


def rows_put(pool: Pool, table: torch.Tensor, seq_len: torch.Tensor, k_new: torch.Tensor,
             v_new: torch.Tensor, max_seq_len: int, ring_pages: int = 0, stream=None):
    """Write k_new/v_new [S][R][Hkv][D] bf16 at positions seq_len - R .. seq_len - 1."""
    S, R = int(k_new.shape[0]), int(k_new.shape[1])
    shape = (S, R, pool.kv_heads, pool.head_dim)
    _need(k_new, torch.bfloat16, "k_new", shape)
    _need(v_new, torch.bfloat16, "v_new", shape)
    lay = _layout(pool, table, seq_len, R, max_seq_len, ring_pages)
    _check(load().kv_rows_put(pool.handle, ctypes.byref(lay), _ptr(k_new), _ptr(v_new), _stream_handle(stream)))


def pages_copy(pool: Pool, src_ids: torch.Tensor, dst_ids: torch.Tensor, stream=None):
    """kv_pages_copy: page dst_ids[i] gets the contents of page src_ids[i] (device int32 [n])."""
    _need(src_ids, torch.int32, "src_ids")
    _need(dst_ids, torch.int32, "dst_ids", tuple(src_ids.shape))
    if src_ids.dim() != 1:
        raise ValueError("src_ids must be 1-D")
    n = int(src_ids.shape[0])
    _check(load().kv_pages_copy(pool.handle, _ptr(src_ids), _ptr(dst_ids), n, _stream_handle(stream)))


def workspace_size(pool: Pool, table: torch.Tensor, seq_len: torch.Tensor, rows: int, q_heads: int,
                   max_seq_len: int, window: int = 0, ring_pages: int = 0) -> int:
    lay = _layout(pool, table, seq_len, rows, max_seq_len, ring_pages)
    args = AttnArgs(None, None, int(q_heads), 0.0, int(window), None, 0)
    n = c_size_t()
    _check(load().paged_attn_workspace_size(pool.handle, ctypes.byref(lay), ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def _attend(entry: str, pool: Pool, q: torch.Tensor, table: torch.Tensor, seq_len: torch.Tensor,
            max_seq_len: int, window: int = 0, ring_pages: int = 0, scale: float = 0.0,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None,
            extra=()):
    if q.dim() != 4 or q.shape[3] != pool.head_dim:
        raise ValueError("q must be [S][R][Hq][D]")
    _need(q, torch.bfloat16, "q")
    S, R, Hq, D = (int(x) for x in q.shape)
    lay = _layout(pool, table, seq_len, R, max_seq_len, ring_pages)
    # buffers this call allocates belong to the stream the kernels run on, so that the caching
    # allocator does not hand their memory to other work before those kernels are done with it
    with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
        if out is None:
            out = torch.empty_like(q)
        if workspace is None:
            nbytes = workspace_size(pool, table, seq_len, R, Hq, max_seq_len, window, ring_pages)
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    _need(out, torch.bfloat16, "out", q.shape)
    args = AttnArgs(_ptr(q), _ptr(out), Hq, float(scale), int(window), _ptr(workspace),
                    int(workspace.numel() * workspace.element_size()))
    _check(getattr(load(), entry)(pool.handle, ctypes.byref(lay), ctypes.byref(args), *extra,
                                  _stream_handle(stream)))
    return out


def decode(pool, q, table, seq_len, max_seq_len, **kw):
    """paged_attn_decode: one row per stream (q [S][1][Hq][D])."""
    return _attend("paged_attn_decode", pool, q, table, seq_len, max_seq_len, **kw)


def decode_put(pool, q, table, seq_len, max_seq_len, k_new: torch.Tensor, v_new: torch.Tensor, **kw):
    """paged_attn_decode_put: write k_new/v_new [S][1][Hkv][D] at position seq_len - 1 and
    decode, in one launch (the same result as rows_put followed by decode)."""
    shape = (int(q.shape[0]), 1, pool.kv_heads, pool.head_dim)
    _need(k_new, torch.bfloat16, "k_new", shape)
    _need(v_new, torch.bfloat16, "v_new", shape)
    return _attend("paged_attn_decode_put", pool, q, table, seq_len, max_seq_len,
                   extra=(_ptr(k_new), _ptr(v_new)), **kw)


STATIC_SCRATCH_BYTES = 32 << 20     # KV_STATIC_SCRATCH_BYTES
KV_MAX_SEQ_LEN = 1 << 29            # the longest max_seq_len and widest window a call may give


def decode_put_static(pool, q, table, seq_len, max_seq_len, k_new: torch.Tensor, v_new: torch.Tensor,
                      window: int = 0, ring_pages: int = 0, scale: float = 0.0, out: torch.Tensor | None = None,
                      stream=None):
    """paged_attn_decode_put_static: paged_attn_decode_put with the library's own per-GPU
    scratch in place of a workspace (no workspace is passed or allocated).  Calls that may run
    at the same time on one GPU race on that scratch."""
    if q.dim() != 4 or q.shape[1] != 1 or q.shape[3] != pool.head_dim:
        raise ValueError("q must be [S][1][Hq][D]")
    _need(q, torch.bfloat16, "q")
    shape = (int(q.shape[0]), 1, pool.kv_heads, pool.head_dim)
    _need(k_new, torch.bfloat16, "k_new", shape)
    _need(v_new, torch.bfloat16, "v_new", shape)
    if out is None:
        if stream is not None:
            with torch.cuda.stream(stream):
                out = torch.empty_like(q)
        else:
            out = torch.empty_like(q)
    _need(out, torch.bfloat16, "out", q.shape)
    lay = _layout(pool, table, seq_len, 1, max_seq_len, ring_pages)
    args = AttnArgs(_ptr(q), _ptr(out), int(q.shape[2]), float(scale), int(window), None, 0)
    _check(load().paged_attn_decode_put_static(pool.handle, ctypes.byref(lay), ctypes.byref(args), _ptr(k_new),
                                               _ptr(v_new), _stream_handle(stream)))
    return out


def verify(pool, q, table, seq_len, max_seq_len, **kw):
    """paged_attn_verify: 1..8 causal rows per stream."""
    return _attend("paged_attn_verify", pool, q, table, seq_len, max_seq_len, **kw)


def verify_tree(pool, q, table, seq_len, max_seq_len, tree_mask: torch.Tensor, **kw):
    """paged_attn_verify_tree: 1..8 rows per stream forming a flattened draft tree;
    tree_mask is a device int32 [S][R] of ancestor bits (bit i of row r: r sees slot i)."""
    _need(tree_mask, torch.int32, "tree_mask", (int(q.shape[0]), int(q.shape[1])))
    return _attend("paged_attn_verify_tree", pool, q, table, seq_len, max_seq_len, extra=(_ptr(tree_mask),), **kw)


def prefill(pool, q, table, seq_len, max_seq_len, **kw):
    """paged_attn_prefill: a prompt chunk of any number of causal rows per stream."""
    return _attend("paged_attn_prefill", pool, q, table, seq_len, max_seq_len, **kw)


def prefill_put(pool, q, table, seq_len, max_seq_len, k_new: torch.Tensor, v_new: torch.Tensor, **kw):
    """paged_attn_prefill_put: write the chunk's rows k_new/v_new [S][R][Hkv][D] at positions
    seq_len - R .. seq_len - 1 and attend (the same result as rows_put followed by prefill)."""
    shape = (int(q.shape[0]), int(q.shape[1]), pool.kv_heads, pool.head_dim)
    _need(k_new, torch.bfloat16, "k_new", shape)
    _need(v_new, torch.bfloat16, "v_new", shape)
    return _attend("paged_attn_prefill_put", pool, q, table, seq_len, max_seq_len,
                   extra=(_ptr(k_new), _ptr(v_new)), **kw)


def set_part_events(start: int | None, stop: int | None):
    """Record the given hipEvent_t handles around the part kernel of later attention calls
    (None, None turns it off)."""
    _check(load().kv_set_part_events(start, stop))


def abi_version() -> int:
    return int(load().kv_abi_version())
