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
  * share(src, dst, n): dst, holding nothing, takes src's first n pages in src's order
    without touching the queue.  A page is then held by several streams; release(stream)
    returns only the pages no other stream still holds, in the releasing stream's order.
    (The Kept states bullet resumes a kept state and reuses its pages; sharing the full pages of
    a common prefix is the form of that which copies nothing.)

A second lease policy, "contiguous", follows the first review of the same PR (its suggestion:
the full layers stay in one unbroken run of pages for as long as the pool has space to spare).  It hands out ids by the first
of these that applies, and removes them from the queue wherever they sit:

  1. extension: the stream holds pages, its newest is t, and t+1, ..., t+n are all free;
  2. placement: among the maximal runs of adjacent free ids with room for n, the longest
     (lowest on a tie), [a, b); the n ids from a if a is 0, else from a + (b - a - n) // 2,
     which leaves half of the run's spare room to the stream that owns page a - 1;
  3. fallback: the n smallest free ids, ascending.

Pins: tests/test_oracle_pins.py checks, against brute-force bookkeeping with sets, that after
any random sequence of leases and releases the leased lists and the free list partition
range(N), no id is leased twice, failed leases change nothing, and hand-out follows the queue;
with shares, that the free list and the union of the leased lists partition range(N), that a
page is free exactly when no list holds it, and a hand-worked sequence of shares and releases.
The contiguous policy is pinned by a hand-worked sequence (tests/golden/contiguous_leases.json)
that reaches each step and the tie rule, and by properties of random sequences: the same
partition, and that every lease is one run of adjacent ids whenever the free set has one.
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
        self.policy = "queue"

    def set_policy(self, policy: str):
        if policy not in ("queue", "contiguous"):
            raise ValueError("policy is 'queue' or 'contiguous'")
        self.policy = policy

    def _free_runs(self):
        """Maximal runs [a, b) of adjacent free ids, in increasing order of a."""
        runs = []
        for i in sorted(self.free):
            if runs and runs[-1][1] == i:
                runs[-1][1] = i + 1
            else:
                runs.append([i, i + 1])
        return [tuple(r) for r in runs]

    def _contiguous_ids(self, stream: int, n: int):
        free = set(self.free)
        mine = self.leased[stream]
        if mine:
            want = [mine[-1] + k for k in range(1, n + 1)]
            if all(i in free for i in want):
                return want
        fits = [(a, b) for a, b in self._free_runs() if b - a >= n]
        if fits:
            longest = max(b - a for a, b in fits)
            a, b = next((a, b) for a, b in fits if b - a == longest)
            start = a if a == 0 else a + (b - a - n) // 2
            return list(range(start, start + n))
        return sorted(free)[:n]

    def lease(self, stream: int, n: int):
        if n < 0 or not (0 <= stream < len(self.leased)):
            raise ValueError("bad stream or count")
        if n > len(self.free):
            raise NoPages(f"{n} pages asked, {len(self.free)} free")
        if self.policy == "queue" or n == 0:
            got = [self.free.popleft() for _ in range(n)]
        else:
            got = self._contiguous_ids(stream, n)
            taken = set(got)
            self.free = deque(i for i in self.free if i not in taken)
        self.leased[stream].extend(got)
        return got

    def holders(self, page: int) -> int:
        """Number of streams whose list holds the page."""
        return sum(page in lst for lst in self.leased)

    def share(self, src: int, dst: int, n: int):
        if not (0 <= src < len(self.leased) and 0 <= dst < len(self.leased)) or src == dst:
            raise ValueError("bad streams")
        if not 0 <= n <= len(self.leased[src]) or self.leased[dst]:
            raise ValueError("bad count, or dst holds pages")
        self.leased[dst] = list(self.leased[src][:n])

    def release(self, stream: int):
        if not (0 <= stream < len(self.leased)):
            raise ValueError("bad stream")
        mine = self.leased[stream]
        self.leased[stream] = []
        self.free.extend(i for i in mine if self.holders(i) == 0)

    @property
    def free_count(self) -> int:
        return len(self.free)
