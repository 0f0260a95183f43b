"""Float64 attention over a linear cache (test infrastructure only).

Definition followed (TensorFold PR #1620; the pages print no formula.  The plainest reading is
taken: the Reads bullet says attention reads its keys through a page table, and the author's
kernel-timing reply says the paged kernels read the very same keys as the linear ones and so
produce identical bits; hence paged attention equals attention over the stream's linear cache):

  For stream s with cache length L (after this call's R rows were written), row r of the call
  sits at position p_r = L - R + r (rows are written before they are read: the Writes bullet
  comes before the Reads bullet).  Query head h reads KV head h // G (heads grouped contiguously;
  the pages give only head counts such as 48/4 and 16/1).  Row r sees keys
  j in [0, p_r] for full layers, or j in [p_r - W + 1, p_r] for a sliding layer of window W
  (W keys including itself; the pages say only that sliding layers keep rings).
      s_j  = scale * <q[s, r, h, :], K[j, h // G, :]>,   scale = 1 / sqrt(d) unless given
      out  = sum_j exp(s_j - max s) V[j, h // G, :] / sum_j exp(s_j - max s)

Verify windows (TensorFold PR #2730: the pending token plus up to seven drafts) are causal
chains of R rows, which is the p_r rule above.

Everything is float64 on values widened exactly from the bf16 inputs.  The per-(stream, KV
head) product is one matrix multiply (a library primitive), the mask is applied by selecting
the visible slice of keys, and the softmax is the textbook max-shifted form.

Pins (tests/test_oracle_pins.py): brute force in pure Python with math.fsum on tiny shapes,
the one-key closed form out = V[0], q = 0 giving the mean of the visible rows, torch's float64
scaled_dot_product_attention with an explicit mask, hand-derived worked examples in
tests/golden/, verify-row == decode-at-that-length, chunked == unchunked prefill,
window >= L == full, and outputs inside the visible rows' range.
"""
import math

import numpy as np


def kv_head_of(h: int, group: int) -> int:
    """Query head h reads KV head h // group (contiguous GQA groups)."""
    return h // group


def row_position(length: int, rows: int, r: int) -> int:
    """Absolute position of row r of a call that leaves the cache at `length`."""
    return length - rows + r


def visible_range(p: int, window: int):
    """Half-open range [lo, hi) of keys that a row at position p attends to."""
    lo = 0 if window <= 0 else max(0, p - window + 1)
    return lo, p + 1


def attend_stream(q, k_lin, v_lin, rows: int, window: int = 0, scale=None, length=None):
    """One stream: q [R][Hq][D] float64, k_lin/v_lin [L][Hkv][D] float64 -> out [R][Hq][D].

    `length` defaults to k_lin.shape[0]; k_lin and v_lin hold positions 0 .. length - 1.  A row
    whose position is negative (more rows than the stream's length, e.g. a stream of length 0)
    sees no key and gets zeros, as a tree row that sees no key does.
    """
    q = np.asarray(q, dtype=np.float64)
    R, Hq, D = q.shape
    Hkv = k_lin.shape[1]
    G = Hq // Hkv
    L = k_lin.shape[0] if length is None else length
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for r in range(R):
        p = row_position(L, R, r)
        lo, hi = visible_range(p, window)
        if hi <= lo:
            continue                                          # a row before the stream
        for kvh in range(Hkv):
            K = k_lin[lo:hi, kvh, :]                          # [n][D]
            V = v_lin[lo:hi, kvh, :]
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            Q = q[r, heads, :]                                # [G][D]
            s = (Q @ K.T) * scale                             # [G][n]
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            out[r, heads, :] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def tree_keys(length: int, rows: int, r: int, mask: int, window: int = 0):
    """Keys that row r of a tree-shaped verify window sees, in increasing order.

    Draft trees (TensorFold PR #1620: decode and drafted verify go through tree attention) are
    flattened into the window's R slots with parents before children; slot i sits at position
    length - rows + i.  Row r sees every key before the window (inside its sliding window, if
    any) and, of the window's own slots, those i <= r whose bit i is set in `mask` (its
    ancestors and itself).  A causal chain is mask = 2^(r+1) - 1.
    """
    p = row_position(length, rows, r)
    lo, hi = visible_range(p, window)
    base = length - rows
    return [j for j in range(lo, hi) if j < base or (mask >> (j - base)) & 1]


def attend_stream_tree(q, k_lin, v_lin, rows: int, masks, window: int = 0, scale=None, length=None):
    """One stream of a tree-shaped verify window: q [R][Hq][D], k_lin/v_lin [L][Hkv][D] float64,
    masks[r] the ancestor bits of row r (see tree_keys).  A row that sees no key gets zeros."""
    q = np.asarray(q, dtype=np.float64)
    R, Hq, D = q.shape
    Hkv = k_lin.shape[1]
    G = Hq // Hkv
    L = k_lin.shape[0] if length is None else length
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((R, Hq, D), dtype=np.float64)
    for r in range(R):
        idx = tree_keys(L, R, r, int(masks[r]), window)
        if not idx:
            continue
        for kvh in range(Hkv):
            K = k_lin[idx, kvh, :]
            V = v_lin[idx, kvh, :]
            heads = [h for h in range(Hq) if kv_head_of(h, G) == kvh]
            s = (q[r, heads, :] @ K.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            w = np.exp(s)
            out[r, heads, :] = (w @ V) / w.sum(axis=1, keepdims=True)
    return out


def attend(q, k_lins, v_lins, lengths, window: int = 0, scale=None):
    """All streams: q [S][R][Hq][D]; k_lins[s], v_lins[s] are [L_s][Hkv][D].  Returns
    out [S][R][Hq][D] float64."""
    q = np.asarray(q, dtype=np.float64)
    S, R = q.shape[:2]
    out = np.empty(q.shape, dtype=np.float64)
    for s in range(S):
        out[s] = attend_stream(q[s], k_lins[s], v_lins[s], R, window, scale, length=lengths[s])
    return out
