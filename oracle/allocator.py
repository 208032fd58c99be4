"""Oracle for the page allocator that keeps the block tables of a paged pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages state: the cache is one pool of pages, and a page table maps
(logical batch, logical block) to a physical page, with pages allocated as
sequences grow and one page per batch slot reserved ahead of a graph
capture so that the in-kernel cache writes hit valid addresses
(benchmarks commit log 1847125, flex_attention paged-KV engine entry,
"Why this works" item 1 and "Files").  They do not state an allocation
policy.  The reading taken here, written as literal stack operations:

* the free pages form a stack ``free_pages[0 .. free_count)`` whose top is
  ``free_pages[free_count - 1]``;
* allocation serves the sequences in batch order and, within a sequence,
  its logical pages in increasing order, each taking the page popped from
  the top of the stack;
* a sequence with ``Lq`` new and ``Lk`` total tokens already holds
  ``ceil((Lk - Lq) / page_size)`` pages and needs ``ceil(Lk / page_size)``;
* the request is all or nothing: when a table row is too short (status 1)
  or the stack holds too few pages (status 2), nothing changes;
* release pushes the pages of each released sequence (``ceil(L /
  page_size)`` of them, logical order, sequences in batch order) and marks
  its table entries -1.
"""
from __future__ import annotations

import numpy as np

ALLOC_OK = 0
ALLOC_TABLE_FULL = 1
ALLOC_OUT_OF_PAGES = 2
FREE_OVERFLOW = 3


def _pages(n_tokens: int, page_size: int) -> int:
    return -(-int(n_tokens) // page_size)


def page_alloc(cu_seq_lens_q, cu_seq_lens_k, block_tables, free_pages, free_count, page_size):
    """Give every sequence the pages its new tokens need.

    Returns ``(block_tables, free_pages, free_count, status)`` as new arrays;
    on a nonzero status they equal the inputs.
    """
    bt = np.array(block_tables, dtype=np.int64, copy=True)
    fp = np.array(free_pages, dtype=np.int64, copy=True)
    stack = [int(p) for p in fp[:free_count]]
    cq = np.asarray(cu_seq_lens_q, dtype=np.int64)
    ck = np.asarray(cu_seq_lens_k, dtype=np.int64)
    plan = []
    for j in range(len(cq) - 1):
        lq, lk = cq[j + 1] - cq[j], ck[j + 1] - ck[j]
        held, want = _pages(lk - lq, page_size), _pages(lk, page_size)
        if want > bt.shape[1]:
            return np.array(block_tables, copy=True), fp, free_count, ALLOC_TABLE_FULL
        plan.append((j, held, want))
    if sum(want - held for _, held, want in plan) > len(stack):
        return np.array(block_tables, copy=True), fp, free_count, ALLOC_OUT_OF_PAGES
    for j, held, want in plan:
        for p in range(held, want):
            bt[j, p] = stack.pop()
    fp[:len(stack)] = stack
    return bt, fp, len(stack), ALLOC_OK


def page_free(seq_lens, release, block_tables, free_pages, free_count, page_size, num_pages):
    """Return the pages of the released sequences to the stack.

    Returns ``(block_tables, free_pages, free_count, status)``; status 3 (and
    nothing changed) if the stack would exceed ``num_pages`` entries.
    """
    bt = np.array(block_tables, dtype=np.int64, copy=True)
    fp = np.array(free_pages, dtype=np.int64, copy=True)
    stack = [int(p) for p in fp[:free_count]]
    back = []
    for j in range(len(seq_lens)):
        if release[j]:
            n = min(_pages(seq_lens[j], page_size), bt.shape[1])
            back += [(j, p) for p in range(n)]
    if len(stack) + len(back) > num_pages:
        return np.array(block_tables, copy=True), fp, free_count, FREE_OVERFLOW
    for j, p in back:
        stack.append(int(bt[j, p]))
        bt[j, p] = -1
    fp[:len(stack)] = stack
    return bt, fp, len(stack), ALLOC_OK
