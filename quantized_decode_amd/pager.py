"""Host-side page allocator for a paged KV pool (bookkeeping only; the pool's
memory and every read and write of it are on the GPU).

P1 "Where it stops, and the argument I got wrong in May": once agents of very
different lengths arrive and finish at different times, the cache is one pool
of fixed-size pages shared by all sequences, and a new sequence is admitted
into the running batch between decode steps.  A pool of n_pages pages of
page_tokens positions is, for the library, a cache layer with n_slots =
n_pages and capacity = page_tokens (include/qkdec.h, paged entry points); the
page table passed to those calls is table(), row b listing sequence b's pages
in logical order.
"""
from __future__ import annotations

from typing import Dict, Iterable, List

import numpy as np


class PagePoolFull(RuntimeError):
    pass


class PagePool:
    def __init__(self, n_pages: int, page_tokens: int):
        if n_pages < 1:
            raise ValueError("n_pages must be >= 1")
        if page_tokens < 32 or page_tokens & (page_tokens - 1):
            raise ValueError("page_tokens must be a power of two >= 32")
        self.n_pages = n_pages
        self.page_tokens = page_tokens
        self._free: List[int] = list(range(n_pages - 1, -1, -1))   # pop() hands out low pages first
        self._pages: Dict[object, List[int]] = {}
        self._len: Dict[object, int] = {}

    # ---- queries
    @property
    def free_pages(self) -> int:
        return len(self._free)

    def pages_for(self, tokens: int) -> int:
        return (max(0, tokens) + self.page_tokens - 1) // self.page_tokens

    def length(self, seq) -> int:
        return self._len[seq]

    def pages(self, seq) -> List[int]:
        return list(self._pages[seq])

    def can_admit(self, tokens: int) -> bool:
        return self.pages_for(tokens) <= self.free_pages

    # ---- changes
    def admit(self, seq, tokens: int) -> List[int]:
        """Give a new sequence pages for `tokens` positions (its prompt plus
        any room wanted ahead)."""
        if seq in self._pages:
            raise KeyError(f"sequence {seq!r} is already admitted")
        need = self.pages_for(tokens)
        if need > self.free_pages:
            raise PagePoolFull(f"{need} pages wanted, {self.free_pages} free")
        self._pages[seq] = [self._free.pop() for _ in range(need)]
        self._len[seq] = max(0, tokens)
        return self.pages(seq)

    def reserve(self, seq, tokens: int) -> List[int]:
        """Grow a sequence to hold `tokens` positions (before a step appends);
        returns the pages added."""
        need = self.pages_for(tokens) - len(self._pages[seq])
        if need > self.free_pages:
            raise PagePoolFull(f"{need} more pages wanted, {self.free_pages} free")
        added = [self._free.pop() for _ in range(max(0, need))]
        self._pages[seq].extend(added)
        self._len[seq] = max(self._len[seq], tokens)
        return added

    def release(self, seq) -> None:
        """A finished sequence returns its pages to the pool."""
        pages = self._pages.pop(seq)
        self._len.pop(seq)
        self._free.extend(reversed(pages))

    def table(self, seqs: Iterable, max_pages: int) -> np.ndarray:
        """int32 [len(seqs), max_pages] page table.  Unused entries are -1, so
        a store into a page the sequence was not given (a step past its
        reserved length) stores nothing and raises the library's capacity
        error instead of writing into another sequence's page."""
        seqs = list(seqs)
        out = np.full((len(seqs), max_pages), -1, dtype=np.int32)
        for b, s in enumerate(seqs):
            p = self._pages[s]
            if len(p) > max_pages:
                raise ValueError(f"sequence {s!r} holds {len(p)} pages, table has {max_pages} columns")
            out[b, :len(p)] = p
        return out
