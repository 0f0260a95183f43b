"""Helpers for the GPU parity tests: run the float64 oracle on the inputs the GPU was given
and compare with the tolerance of bf16 inputs and fp32 accumulation.

Expected values never come from the HIP path.  The oracle's inputs are the seeded generator's
values (queries, and each stream's K/V history as written) and the host copy of the page
table; where a test needs the whole pool as the library should have left it, `expected_pool`
builds it on the host with the oracle's own scatter over a pool filled with the NaN pattern.
"""
import math

import numpy as np
import torch

import oracle
from paged_kv_cache_rows_amd import binding, staging, workloads

# The bound for bf16 inputs with fp32 accumulation: max-abs 2e-2 and relative 1e-2, read as
# max |gpu - oracle| <= 2e-2 over the output, and relative L2 error
# ||gpu - oracle|| / ||oracle|| <= 1e-2, over the whole output and over each stream's part.
ATOL = 2e-2
REL_L2 = 1e-2


def say(msg: str):
    print(msg, flush=True)


def pool_bits(cache):
    """(K bits, V bits) of the whole GPU pool on the host, uint16 [N][Hkv][P][D]."""
    return workloads.bf16_bits(cache.pool.k_pages), workloads.bf16_bits(cache.pool.v_pages)


def host_history(ks, vs):
    """Host bf16 copies of per-stream histories (device or host tensors)."""
    return [k.detach().cpu() for k in ks], [v.detach().cpu() for v in vs]


def remember(cache, ks, vs, upto=None):
    """Record on the cache the rows written so far (the generator's values), which the oracle
    reads instead of the GPU pool."""
    ks, vs = host_history(ks, vs)
    n = cache.lengths if upto is None else upto
    cache.history = ([k[:L] for k, L in zip(ks, n)], [v[:L] for v, L in zip(vs, n)])
    return cache


def expected_pool(cache, fill_bits=workloads.NAN_BITS):
    """The pool the row writes should leave, built on the host by the oracle: every page filled
    with the NaN pattern, then each stream's recorded history scattered through its table."""
    w = cache.w
    shape = (w.pool_pages, w.kv_heads, w.page_size, w.head_dim)
    kb = np.full(shape, fill_bits, dtype=np.uint16)
    vb = np.full(shape, fill_bits, dtype=np.uint16)
    ks, vs = cache.history
    for s in range(w.streams):
        L = ks[s].shape[0]
        if L == 0:
            continue
        kb = oracle.rows_put(kb, cache.table_host[s], L, workloads.bf16_bits(ks[s]), w.page_size, cache.ring_pages)
        vb = oracle.rows_put(vb, cache.table_host[s], L, workloads.bf16_bits(vs[s]), w.page_size, cache.ring_pages)
    return kb, vb


def oracle_for(cache, q: torch.Tensor, window: int = 0, streams=None, lengths=None, scale=None):
    """Oracle output [S'][R][Hq][D] float64 for the selected streams, from the generator's
    history recorded on the cache (the linear cache each stream wrote)."""
    ks, vs = cache.history
    lengths = cache.lengths if lengths is None else lengths
    streams = range(cache.w.streams) if streams is None else streams
    return oracle_from_history(ks, vs, q, lengths, window, streams=streams, scale=scale)


def oracle_tree_for(cache, q: torch.Tensor, masks, window: int = 0):
    """Oracle output [S][R][Hq][D] of a tree-shaped verify window (masks [S][R] ancestor bits),
    from the history recorded on the cache."""
    ks, vs = cache.history
    qb = workloads.bf16_bits(q)
    outs = []
    for s in range(cache.w.streams):
        L = cache.lengths[s]
        kl = oracle.bf16_bits_to_f64(workloads.bf16_bits(ks[s][:L]))
        vl = oracle.bf16_bits_to_f64(workloads.bf16_bits(vs[s][:L]))
        qs = oracle.bf16_bits_to_f64(qb[s])
        outs.append(oracle.attend_stream_tree(qs, kl, vl, qs.shape[0], [int(m) for m in masks[s]], window,
                                              length=L))
    return np.stack(outs)


def random_tree_masks(rng, streams: int, rows: int):
    """Ancestor bits [S][R] of random draft trees, parents before children (parent[i] < i)."""
    out = np.zeros((streams, rows), dtype=np.int64)
    for s in range(streams):
        parent = [-1] + [int(rng.integers(0, i)) for i in range(1, rows)]
        for r in range(rows):
            m, i = 0, r
            while i >= 0:
                m |= 1 << i
                i = parent[i]
            out[s, r] = m
    return out


def oracle_from_history(ks, vs, q: torch.Tensor, lengths, window=0, streams=None, scale=None):
    """Oracle output from history tensors (the rows each stream wrote, positions 0..L-1):
    attention over the linear cache."""
    qb = workloads.bf16_bits(q)
    streams = range(len(lengths)) if streams is None else streams
    outs = []
    for s in streams:
        L = lengths[s]
        kl = oracle.bf16_bits_to_f64(workloads.bf16_bits(ks[s][:L]))
        vl = oracle.bf16_bits_to_f64(workloads.bf16_bits(vs[s][:L]))
        qs = oracle.bf16_bits_to_f64(qb[s])
        outs.append(oracle.attend_stream(qs, kl, vl, qs.shape[0], window, scale=scale, length=L))
    return np.stack(outs)


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(workloads.bf16_bits(t))


def _rel(d: np.ndarray, r: np.ndarray) -> float:
    nr = float(np.linalg.norm(r))
    nd = float(np.linalg.norm(d))
    if nr == 0.0:
        return 0.0 if nd == 0.0 else math.inf
    return nd / nr


def compare(gpu, ref: np.ndarray):
    """(ok, max_abs, rel_l2, worst_index, worst_stream_rel) of gpu against the oracle: ok when
    every value is finite, max |g - o| <= ATOL, and the relative L2 error is <= REL_L2 over the
    whole output and over each stream's slice (axis 0; an all-zero reference slice needs an
    all-zero output)."""
    g = gpu_f64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert g.shape == ref.shape, (g.shape, ref.shape)
    finite = bool(np.isfinite(g).all())
    d = np.where(np.isfinite(g), g - ref, np.inf)
    err = np.abs(d)
    mx = float(err.max()) if err.size else 0.0
    rel = _rel(np.where(np.isfinite(d), d, 0.0), ref) if finite else math.inf
    per = [_rel(d[s], ref[s]) if finite else math.inf for s in range(g.shape[0])] if g.ndim > 1 else [rel]
    worst_stream = max(per) if per else 0.0
    ok = finite and mx <= ATOL and rel <= REL_L2 and worst_stream <= REL_L2
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else ()
    return ok, mx, rel, tuple(int(i) for i in worst), worst_stream


def assert_close(gpu, ref, what=""):
    ok, mx, rel, worst, per = compare(gpu, ref)
    say(f"  {what}: max_abs {mx:.3e} rel_l2 {rel:.3e} worst stream rel_l2 {per:.3e}")
    assert ok, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e} worst stream rel_l2 {per:.3e} worst at {worst}"


def assert_red(gpu, ref, what=""):
    """A control: the comparison must fail."""
    ok, mx, rel, worst, per = compare(gpu, ref)
    say(f"  control {what}: max_abs {mx:.3e} rel_l2 {rel:.3e} worst stream rel_l2 {per:.3e} -> "
        f"{'GREEN (not detected)' if ok else 'red'}")
    assert not ok, f"control {what} was not detected: max_abs {mx:.3e} rel_l2 {rel:.3e}"


def new_cache(w, order_seed=None, identity=False, fill_bits=workloads.NAN_BITS, history=True,
              device="cuda", lengths=None, salt=0):
    """A cache for w with its history written; returns (cache, ks, vs) with histories on the
    host (bf16 CPU tensors).  The cache records the history for the oracle."""
    if identity:
        order = workloads.identity_order(w.pool_pages)
    else:
        order = workloads.free_order(w.pool_pages, w.seed + 2000 if order_seed is None else order_seed)
    c = staging.make_cache(w, device=device, order=order, fill_bits=fill_bits, lengths=lengths)
    ks = vs = None
    if history:
        wl = w if lengths is None else _with_lengths(w, lengths)
        ks, vs = workloads.kv_history(wl, device="cpu", salt=salt)
        staging.write_history(c, ks, vs)
        remember(c, ks, vs)
    return c, ks, vs


def _with_lengths(w, lengths):
    import dataclasses
    return dataclasses.replace(w, lengths=list(lengths))


def poisoned_workspace(cache, rows, q_heads, window=0):
    """A workspace filled with NaN bytes, so a read of any partial the kernels did not write
    shows up in the output."""
    n = binding.workspace_size(cache.pool, cache.table, cache.seq_len, rows, q_heads, cache.max_seq_len,
                               window, cache.ring_pages)
    return torch.full((max(n, 256),), 0xFF, dtype=torch.uint8, device=cache.table.device)


def attend(entry, cache, q, window=0, **kw):
    fn = {"decode": binding.decode, "verify": binding.verify, "prefill": binding.prefill}[entry]
    if "workspace" not in kw:
        kw["workspace"] = poisoned_workspace(cache, q.shape[1], q.shape[2], window)
    out = fn(cache.pool, q, cache.table, cache.seq_len, cache.max_seq_len, window=window,
             ring_pages=cache.ring_pages, **kw)
    torch.cuda.synchronize()
    return out
