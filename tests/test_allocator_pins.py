"""Pins for the page-allocator oracle: a worked example derived by hand
(tests/golden/page_alloc.txt) and invariants that any correct allocator
keeps (every page owned at most once and either owned or free, coverage of
every sequence's tokens, all-or-nothing failures, last-in-first-out reuse)."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_alloc.txt")


def _ints(text):
    return [int(x) for x in text.split()]


def _golden():
    lines = [ln.split("#", 1)[0].strip() for ln in open(GOLDEN)]
    return [ln for ln in lines if ln]


def test_worked_example():
    lines = _golden()
    kv = {}
    i = 0
    while "/" not in lines[i]:   # header: "key values"; steps carry "/" separators
        key, rest = lines[i].split(" ", 1)
        kv[key] = _ints(rest)
        i += 1
    ps, num_pages = kv["page_size"][0], kv["num_pages"][0]
    nseq, width = kv["table"]
    bt = np.full((nseq, width), -1, np.int64)
    free = np.array(kv["free"], np.int64)
    count = len(free)
    steps = lines[i:]
    assert len(steps) % 2 == 0
    for op, exp in zip(steps[0::2], steps[1::2]):
        name, rest = op.split(" ", 1)
        a, b = [_ints(x) for x in rest.split("/")]
        if name == "alloc":
            cq = np.concatenate([[0], np.cumsum(a)])
            ck = np.concatenate([[0], np.cumsum(b)])
            bt, free, count, st = oracle.page_alloc(cq, ck, bt, free, count, ps)
        else:
            bt, free, count, st = oracle.page_free(a, b, bt, free, count, ps, num_pages)
        parts = exp.split(" ", 1)[1].split("/")
        assert st == int(parts[0]), op
        if parts[1].strip() != "-":
            assert list(free[:count]) == _ints(parts[1]), op
        else:
            assert count == 0, op
        rows = [_ints(r) for r in parts[2:]]
        assert bt.tolist() == rows, op


def _owned(bt, lens, ps):
    out = []
    for j, L in enumerate(lens):
        out += [int(p) for p in bt[j, :-(-int(L) // ps)]]
    return out


@pytest.mark.parametrize("seed", range(6))
def test_invariants_random(seed):
    rng = np.random.default_rng(seed)
    ps, width, nseq, num_pages = 16, 6, 5, 20
    bt = np.full((nseq, width), -1, np.int64)
    free = rng.permutation(num_pages).astype(np.int64)
    count = num_pages
    lens = np.zeros(nseq, np.int64)
    for _ in range(40):
        if rng.random() < 0.7:
            lq = rng.integers(0, 40, nseq) * (rng.random(nseq) < 0.7)
            lk = lens + lq
            before = (bt.copy(), free.copy(), count)
            bt, free, count, st = oracle.page_alloc(np.concatenate([[0], np.cumsum(lq)]),
                                                    np.concatenate([[0], np.cumsum(lk)]),
                                                    bt, free, count, ps)
            need = sum(-(-int(k) // ps) - -(-int(k - q) // ps) for q, k in zip(lq, lk))
            if st == oracle.ALLOC_OK:
                lens = lk
                assert count == before[2] - need
                # the taken pages are the top of the old stack, in pop order
                taken = [int(bt[j, p]) for j in range(nseq)
                         for p in range(-(-int(lk[j] - lq[j]) // ps), -(-int(lk[j]) // ps))]
                assert taken == [int(x) for x in before[1][:before[2]][::-1][:need]]
            else:
                assert np.array_equal(bt, before[0]) and count == before[2]
                assert np.array_equal(free, before[1])
                if st == oracle.ALLOC_TABLE_FULL:
                    assert any(-(-int(k) // ps) > width for k in lk)
                else:
                    assert st == oracle.ALLOC_OUT_OF_PAGES and need > before[2]
        else:
            rel = (rng.random(nseq) < 0.4).astype(np.int64)
            bt, free, count, st = oracle.page_free(lens, rel, bt, free, count, ps, num_pages)
            assert st == oracle.ALLOC_OK
            assert np.all(bt[rel.astype(bool)] == -1)
            lens = np.where(rel.astype(bool), 0, lens)
        owned = _owned(bt, lens, ps)
        pool = owned + [int(p) for p in free[:count]]
        assert sorted(pool) == list(range(num_pages))       # conservation, no duplicate


def test_lifo_reuse():
    # freeing n pages and then allocating n pages for a fresh sequence hands
    # the same pages back in reverse order of the release
    ps = 8
    bt = np.array([[3, 9, 4], [-1, -1, -1]], np.int64)
    free = np.array([0, 1, 2, 5, 6, 7, 8, 0, 0, 0], np.int64)
    bt, free, count, st = oracle.page_free([20, 0], [1, 0], bt, free, 7, ps, 10)
    assert st == 0 and count == 10 and list(free[7:10]) == [3, 9, 4]
    bt, free, count, st = oracle.page_alloc([0, 0, 24], [0, 0, 24], bt, free, count, ps)
    assert st == 0 and count == 7 and bt[1].tolist() == [4, 9, 3]


def test_free_overflow_is_refused():
    bt = np.array([[1, 2]], np.int64)
    free = np.arange(4, dtype=np.int64)
    out = oracle.page_free([9], [1], bt, free, 3, 8, 4)   # 3 free + 2 back > 4 pages
    assert out[3] == oracle.FREE_OVERFLOW and out[2] == 3 and out[0].tolist() == [[1, 2]]
