"""The oracle's own walk of the page table (test infrastructure only).

Pool layout (this library's choice; the pages do not fix one): K and V pages are arrays
[num_pages][Hkv][P][D] of bf16, so one KV head's rows inside a page are contiguous.

TensorFold PR #1620, opening description: pages of 512 positions leased from the core pool,
the Writes bullet (new rows copied into their page slots) and the Reads bullet (keys read through
a per-stream page table in the call's stream order); sliding layers keep rings.  Positions map to slots as:
    full layer:  page = table[j // P],                  slot = j % P
    ring layer:  page = table[(j // P) % ring_pages],   slot = j % P
so a ring of n pages holds the newest n*P positions.

Pins: gather_linear(rows_put(...)) returns exactly the rows written (a round trip checked on
random tables, page sizes 1, 3, 37, 64, 512 and rings), gather over a shuffled pool equals the
gather over an identity pool bit for bit, and slot_of is compared with brute-force enumeration
of positions in tests/test_oracle_pins.py.
"""
import numpy as np


def slot_of(j: int, table_row, page_size: int, ring_pages: int = 0):
    """(physical page, slot) holding position j of a stream."""
    idx = j // page_size
    if ring_pages:
        idx %= ring_pages
    return int(table_row[idx]), j % page_size


def gather_linear(pages, table_row, length: int, page_size: int, ring_pages: int = 0):
    """Rebuild a stream's linear cache [L][Hkv][D] from pages [N][Hkv][P][D].

    For a ring, only the newest ring_pages * page_size positions still exist; returns
    (array, first_position) in that case, else just the array starting at position 0.
    """
    pages = np.asarray(pages)
    _, Hkv, P, D = pages.shape
    assert P == page_size
    first = 0
    if ring_pages:
        first = max(0, length - ring_pages * page_size)
    out = np.empty((length - first, Hkv, D), dtype=pages.dtype)
    # One logical page at a time: positions [idx*P, (idx+1)*P) share one table entry.
    for idx in range(first // page_size, -(-length // page_size)):
        j0 = max(idx * page_size, first)
        j1 = min((idx + 1) * page_size, length)
        pg, sl0 = slot_of(j0, table_row, page_size, ring_pages)
        out[j0 - first:j1 - first] = pages[pg, :, sl0:sl0 + (j1 - j0), :].transpose(1, 0, 2)
    if ring_pages:
        return out, first
    return out


def rows_put(pages, table_row, length: int, rows_new, page_size: int, ring_pages: int = 0):
    """Return a copy of pages [N][Hkv][P][D] with rows_new [R][Hkv][D] written at positions
    length - R .. length - 1 of the stream (R = rows_new.shape[0])."""
    out = np.array(pages, copy=True)
    R = rows_new.shape[0]
    for r in range(R):
        j = length - R + r
        pg, sl = slot_of(j, table_row, page_size, ring_pages)
        out[pg, :, sl, :] = rows_new[r]
    return out


def copy_pages(pages, src_ids, dst_ids, num_pages=None):
    """Return a copy of pages [N][Hkv][P][D] in which page dst_ids[i] holds what page src_ids[i]
    held, for every i whose two ids are inside the pool (kept states: a stream's state is kept
    by copying the pages its table lists, opening description, Kept states bullet).  Copies
    are taken from the pages as they were before any copy of the call."""
    src = np.asarray(pages)
    out = np.array(src, copy=True)
    n = src.shape[0] if num_pages is None else num_pages
    for a, b in zip(src_ids, dst_ids):
        if 0 <= int(a) < n and 0 <= int(b) < n:
            out[int(b)] = src[int(a)]
    return out
