"""TEST INFRASTRUCTURE ONLY.  Reference (oracle) model of dynamic optional
residency: which pages of each request's imported history are held in the
device pool, which of them are ready, and how admission, completion and
repopulation change that.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this module; the product library never calls it.

Source: "Adaptive DHiSparse: Speculative Decoding over a Load-Adaptive KV
Hierarchy" (arXiv 2610.13708):
  - §3.1 "Load-Adaptive Residency", eq. (3): required allocations, optional
    history and the admission reserve together stay within the pool capacity M.
  - §3.1, eq. (4): an admission that leaves a deficit of Delta pages reclaims
    whole requests, walking the reclaim order and taking the first q whose
    optional pages cover Delta; the others keep their pages; if nothing covers
    Delta the admission waits.
  - §3.1: optional residency covers complete pages of a request's imported
    history; rows generated while decoding and the partial boundary page stay
    with the tail and hot cache.  Population reserves pages, copies their
    rows and publishes them as ready only after the copy; a pending page is
    invisible to resolution.  A bounded round-robin scheduler repopulates a
    limited number of pages per attempt.  Completion releases the request's
    capacity.
  - Figure 2 / §3.2: resolution consults the ready optional map first.

Readings where the pages leave a step open (one numbering R1-R27 covers
every reading taken of the pages; R1-R10, R24, R26 and R27 are in ``model.py``):
  R17 the pool holds M pages of P rows; an admitted request's required
      allocations (hot cache, tail, staging) are charged against M in pages
      but occupy no pool page; optional pages occupy pool pages.  Eq. (3)
      is the invariant  sum(required) + sum(held) + reserve <= M.
  R18 eligible pages of a request are floor(n_r / P) for its frontier n_r
      at admission (complete pages of the imported history).
  R19 a_r of eq. (4) counts every page the request holds, pending or ready;
      the reclaim order is the caller's policy and is passed with the
      admission; reclaiming a request drops all of its optional pages
      (pending or ready) and leaves it admitted and eligible for later
      repopulation; if the whole order cannot cover the deficit the admission
      waits and nothing changes.
  R20 one population attempt visits request slots cyclically from a cursor
      that persists between attempts; a visit to an admitted request that
      holds fewer than its eligible pages assigns its lowest page index not
      held to the lowest free pool page; the attempt ends after max_pages
      assignments, when the budget M - sum(required) - reserve - sum(held) is
      used up, or after a whole cycle with no assignment; the cursor then
      points past the last visited slot.
  R21 a page becomes ready (visible to resolution) only when it is published
      after its copy has completed.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple


class OptResidency:
    """Pool of `pool_pages` pages of `page_rows` rows, shared by every layer
    group (one decision per request covers all of its layers)."""

    def __init__(self, n_req: int, pool_pages: int, page_rows: int, reserve: int):
        if n_req <= 0 or pool_pages < 0 or page_rows <= 0 or reserve < 0:
            raise ValueError("bad residency sizes")
        self.N = n_req
        self.M = pool_pages
        self.P = page_rows
        self.reserve = reserve
        self.admitted = [False] * n_req
        self.required = [0] * n_req
        self.eligible = [0] * n_req
        self.held: List[Dict[int, int]] = [dict() for _ in range(n_req)]   # page index -> pool page
        self.ready: List[set] = [set() for _ in range(n_req)]              # page indexes published
        self.free = set(range(pool_pages))
        self.cursor = 0

    # ------------------------------------------------------------- accounting
    def sum_required(self) -> int:
        return sum(self.required)

    def sum_held(self) -> int:
        return sum(len(h) for h in self.held)

    def budget(self) -> int:
        """Pages population may still take under eq. (3)."""
        return self.M - self.sum_required() - self.reserve - self.sum_held()

    # ------------------------------------------------------------- transitions
    def _drop(self, r: int):
        for pool in self.held[r].values():
            self.free.add(pool)
        self.held[r] = {}
        self.ready[r] = set()

    def admit(self, r: int, n_r: int, required_pages: int, order: Sequence[int]) -> Optional[List[int]]:
        """Admission of request r (eq. 3, eq. 4).  Returns the reclaimed
        requests r_1..r_q, or None when the admission has to wait (no change)."""
        if self.admitted[r]:
            raise ValueError("request already admitted")
        if required_pages < 0:
            raise ValueError("negative required pages")
        order = [int(x) for x in order]
        if len(set(order)) != len(order) or any(not self.admitted[x] for x in order):
            raise ValueError("reclaim order must list distinct admitted requests")
        deficit = self.sum_required() + required_pages + self.sum_held() + self.reserve - self.M
        taken: List[int] = []
        if deficit > 0:
            covered = 0
            for x in order:                       # eq. (4): the first q with sum a >= Delta
                if covered >= deficit:
                    break
                taken.append(x)
                covered += len(self.held[x])
            if covered < deficit:
                return None                       # the admission waits
        for x in taken:
            self._drop(x)
        self.admitted[r] = True
        self.required[r] = required_pages
        self.eligible[r] = max(0, n_r) // self.P  # R18
        return taken

    def complete(self, r: int):
        """Completion releases the request's required and optional capacity."""
        if not self.admitted[r]:
            raise ValueError("request not admitted")
        self._drop(r)
        self.admitted[r] = False
        self.required[r] = 0
        self.eligible[r] = 0

    def populate(self, max_pages: int) -> List[Tuple[int, int, int]]:
        """One bounded round-robin attempt (R20).  Returns the new pending
        pages as (request, page index, pool page), in assignment order."""
        if max_pages < 0:
            raise ValueError("negative page bound")
        limit = min(max_pages, self.budget())
        out: List[Tuple[int, int, int]] = []
        r = self.cursor
        idle = 0
        while len(out) < limit and idle < self.N:
            if self.admitted[r] and len(self.held[r]) < self.eligible[r]:
                idx = next(i for i in range(self.eligible[r]) if i not in self.held[r])
                pool = min(self.free)
                self.free.remove(pool)
                self.held[r][idx] = pool
                out.append((r, idx, pool))
                idle = 0
            else:
                idle += 1
            r = (r + 1) % self.N
        self.cursor = r
        return out

    def publish(self, pages: Optional[Sequence[Tuple[int, int, int]]] = None):
        """Copies complete: pending pages become ready (all of them, or the
        listed ones that are still held by the same request)."""
        if pages is None:
            for r in range(self.N):
                self.ready[r] = set(self.held[r])
            return
        for r, idx, pool in pages:
            if self.held[r].get(idx) == pool:
                self.ready[r].add(idx)

    # ------------------------------------------------------------- views
    def lookup(self, r: int, row: int) -> Optional[int]:
        """Resident pool row of history row `row` of request r if its page is
        ready (Figure 2 callout 1), else None."""
        idx = row // self.P
        if idx in self.ready[r]:
            return self.held[r][idx] * self.P + row % self.P
        return None

    def page_table(self, r: int, n_pages: int) -> Tuple[List[int], List[int]]:
        """Pool page held for each page index (-1 none) and whether it is ready."""
        held = [self.held[r].get(i, -1) for i in range(n_pages)]
        ready = [1 if i in self.ready[r] else 0 for i in range(n_pages)]
        return held, ready

    def coverage(self) -> Tuple[int, int]:
        """Ready pages and eligible pages over admitted requests (Figure 6b)."""
        return (sum(len(self.ready[r]) for r in range(self.N) if self.admitted[r]),
                sum(self.eligible[r] for r in range(self.N) if self.admitted[r]))
