"""Plain Python model of the shared page pool (test infrastructure only).

TensorFold PR #1620, opening description: the full layers' caches live in pages of one core
pool and every stream leases pages as it grows; the Kept states bullet and the model test
say released pages are handed out again.  The pages give no hand-out order,
so this library fixes one and the model states it:

  * The free list is a FIFO queue, initialised with `free_order` (default 0, 1, ..., N-1).
  * lease(stream, n) takes the first n ids of the queue, in queue order, and appends them to
    the stream's page list.  If fewer than n are free it fails and changes nothing.
  * release(stream) appends the stream's pages to the back of the queue in the order they
    were leased, and empties the stream's list.

Pins: tests/test_oracle_pins.py checks, against brute-force bookkeeping with sets, that after
any random sequence of leases and releases the leased lists and the free list partition
range(N), no id is leased twice, failed leases change nothing, and hand-out follows the queue.
"""
from collections import deque


class NoPages(Exception):
    pass


class LeaseModel:
    def __init__(self, num_pages: int, max_streams: int, free_order=None):
        order = list(range(num_pages)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_pages)):
            raise ValueError("free_order must be a permutation of the page ids")
        self.num_pages = num_pages
        self.free = deque(order)
        self.leased = [[] for _ in range(max_streams)]

    def lease(self, stream: int, n: int):
        if n < 0 or not (0 <= stream < len(self.leased)):
            raise ValueError("bad stream or count")
        if n > len(self.free):
            raise NoPages(f"{n} pages asked, {len(self.free)} free")
        got = [self.free.popleft() for _ in range(n)]
        self.leased[stream].extend(got)
        return got

    def release(self, stream: int):
        if not (0 <= stream < len(self.leased)):
            raise ValueError("bad stream")
        self.free.extend(self.leased[stream])
        self.leased[stream] = []

    @property
    def free_count(self) -> int:
        return len(self.free)
