"""Helpers for the GPU parity tests: copy the GPU's pool and tables to the host, run the
float64 oracle on them, and compare with the tolerance of bf16 inputs and fp32 accumulation.

The oracle side sees only host copies of what the GPU was given (bf16 bit patterns, page ids,
lengths); nothing computed by the HIP path feeds an expected value.
"""
import math

import numpy as np
import torch

import oracle
from paged_kv_cache_rows_amd import binding, staging, workloads

ATOL = 2e-2   # elementwise |gpu - oracle| <= ATOL + RTOL * |oracle|
RTOL = 1e-2


def say(msg: str):
    print(msg, flush=True)


def pool_bits(cache):
    """(K bits, V bits) of the whole pool on the host, uint16 [N][Hkv][P][D]."""
    return workloads.bf16_bits(cache.pool.k_pages), workloads.bf16_bits(cache.pool.v_pages)


def oracle_for(cache, q: torch.Tensor, window: int = 0, streams=None, kbits=None, vbits=None,
               lengths=None, scale=None):
    """Oracle output [S'][R][Hq][D] float64 for the selected streams, gathering each stream's
    linear cache from host copies of the GPU pool through the oracle's own table walk."""
    if kbits is None:
        kbits, vbits = pool_bits(cache)
    lengths = cache.lengths if lengths is None else lengths
    streams = range(cache.w.streams) if streams is None else streams
    qb = workloads.bf16_bits(q)
    outs = []
    for s in streams:
        L = lengths[s]
        kl = oracle.gather_linear(kbits, cache.table_host[s], L, cache.w.page_size, cache.ring_pages)
        vl = oracle.gather_linear(vbits, cache.table_host[s], L, cache.w.page_size, cache.ring_pages)
        if cache.ring_pages:
            kl = (oracle.bf16_bits_to_f64(kl[0]), kl[1])
            vl = (oracle.bf16_bits_to_f64(vl[0]), vl[1])
        else:
            kl, vl = oracle.bf16_bits_to_f64(kl), oracle.bf16_bits_to_f64(vl)
        qs = oracle.bf16_bits_to_f64(qb[s])
        outs.append(oracle.attend_stream(qs, kl, vl, qs.shape[0], window, scale=scale, length=L))
    return np.stack(outs)


def oracle_tree_for(cache, q: torch.Tensor, masks, window: int = 0):
    """Oracle output [S][R][Hq][D] of a tree-shaped verify window (masks [S][R] ancestor bits),
    gathering each stream's linear cache from host copies of the GPU pool."""
    kbits, vbits = pool_bits(cache)
    qb = workloads.bf16_bits(q)
    outs = []
    for s in range(cache.w.streams):
        L = cache.lengths[s]
        kl = oracle.bf16_bits_to_f64(oracle.gather_linear(kbits, cache.table_host[s], L, cache.w.page_size))
        vl = oracle.bf16_bits_to_f64(oracle.gather_linear(vbits, cache.table_host[s], L, cache.w.page_size))
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


def oracle_from_history(ks, vs, q: torch.Tensor, lengths, window=0, streams=None):
    """Oracle output from the generator's history tensors directly (for ring layers, whose
    pool no longer holds the old positions)."""
    qb = workloads.bf16_bits(q)
    streams = range(len(lengths)) if streams is None else streams
    outs = []
    for s in streams:
        L = lengths[s]
        kl = oracle.bf16_bits_to_f64(workloads.bf16_bits(ks[s][:L]))
        vl = oracle.bf16_bits_to_f64(workloads.bf16_bits(vs[s][:L]))
        qs = oracle.bf16_bits_to_f64(qb[s])
        outs.append(oracle.attend_stream(qs, kl, vl, qs.shape[0], window, length=L))
    return np.stack(outs)


def gpu_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(workloads.bf16_bits(t))


def compare(gpu: torch.Tensor, ref: np.ndarray):
    """(ok, max_abs, rel_l2, worst_index) under |g - o| <= ATOL + RTOL |o|."""
    g = gpu_f64(gpu) if isinstance(gpu, torch.Tensor) else gpu
    assert g.shape == ref.shape, (g.shape, ref.shape)
    err = np.abs(g - ref)
    bound = ATOL + RTOL * np.abs(ref)
    ok = bool(np.isfinite(g).all() and (err <= bound).all())
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    return ok, float(np.nanmax(err)), rel, tuple(int(i) for i in worst)


def assert_close(gpu, ref, what=""):
    ok, mx, rel, worst = compare(gpu, ref)
    say(f"  {what}: max_abs {mx:.3e} rel_l2 {rel:.3e}")
    assert ok, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e} worst at {worst}"


def new_cache(w, order_seed=None, identity=False, fill_bits=workloads.NAN_BITS, history=True,
              device="cuda", lengths=None, salt=0):
    """A cache for w with its history written; returns (cache, ks, vs) with histories on the
    host (bf16 CPU tensors)."""
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
