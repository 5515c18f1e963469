"""Plain model of the page allocator (TEST INFRASTRUCTURE ONLY; shares nothing with the library).

"Fitting a 27B-Parameter LLM into 24 GiB of Laptop Memory", section "StateTrans: Request
Transitions at Safe Boundaries": admission reserves physical-page equivalents, the ceiling of
(prompt length + min(output budget, 8,192)) over the 256-token page size; shared prefixes use
reference counts; completion filters departing rows and only then drops page references, and a
page returns to the free list when its count reaches zero after that boundary.

Readings (the page gives no more): the free list is first in, first out, starting with all page
IDs in ascending order; reservations are a budget that all live requests' reservations must fit;
growth past a request's reservation takes free pages while any remain; shared prefix pages are
whole pages already held by a live request."""
from __future__ import annotations

from collections import deque

GUARANTEED_OUTPUT = 8192


def admission_need(prompt_len: int, output_budget: int, page_size: int) -> int:
    tokens = prompt_len + min(output_budget, GUARANTEED_OUTPUT)
    return -(-tokens // page_size)


class PagePool:
    def __init__(self, num_pages: int, page_size: int):
        self.num_pages, self.page_size = num_pages, page_size
        self.refcount = [0] * num_pages
        self.free = deque(range(num_pages))
        self.reserved = 0
        self.requests = []          # [reservation, pages, live, departing]
        self.departing = []

    def admit(self, prompt_len, output_budget, prefix_pages=()):
        need = admission_need(prompt_len, output_budget, self.page_size)
        if len(prefix_pages) * self.page_size > prompt_len:
            raise ValueError("prefix longer than the prompt")
        if any(self.refcount[p] < 1 for p in prefix_pages):
            raise ValueError("a shared page is not held")
        if self.reserved + need > self.num_pages:
            return None
        for p in prefix_pages:
            self.refcount[p] += 1
        self.reserved += need
        self.requests.append([need, list(prefix_pages), True, False])
        return len(self.requests) - 1

    def extend(self, rid, length):
        r = self.requests[rid]
        assert r[2] and not r[3]
        more = -(-length // self.page_size) - len(r[1])
        if more <= 0:
            return True
        if more > len(self.free):
            return False
        for _ in range(more):
            p = self.free.popleft()
            self.refcount[p] = 1
            r[1].append(p)
        return True

    def table(self, rid):
        return list(self.requests[rid][1])

    def finish(self, rid):
        r = self.requests[rid]
        assert r[2] and not r[3]
        r[3] = True
        self.departing.append(rid)

    def boundary(self):
        for rid in self.departing:
            r = self.requests[rid]
            for p in r[1]:
                self.refcount[p] -= 1
                if self.refcount[p] == 0:
                    self.free.append(p)
            self.reserved -= r[0]
            r[1], r[2] = [], False
        self.departing = []
