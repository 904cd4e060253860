"""Host page allocator of the paged KV pool."""
import numpy as np
import pytest

from quantized_decode_amd.pager import PagePool, PagePoolFull


def test_admit_grow_release_and_table():
    pool = PagePool(8, 64)
    assert pool.admit("a", 100) == [0, 1]
    assert pool.admit("b", 1) == [2]
    assert pool.reserve("b", 64) == [] and pool.reserve("b", 65) == [3]
    assert pool.length("b") == 65 and pool.free_pages == 4
    t = pool.table(["b", "a"], 4)
    assert t.dtype == np.int32 and t.tolist() == [[2, 3, -1, -1], [0, 1, -1, -1]]
    pool.release("a")
    assert pool.free_pages == 6
    assert pool.admit("c", 128) == [0, 1]            # freed pages are reused
    with pytest.raises(PagePoolFull):
        pool.admit("d", 5 * 64)
    assert pool.can_admit(4 * 64) and not pool.can_admit(4 * 64 + 1)
    with pytest.raises(KeyError):
        pool.admit("c", 1)
    with pytest.raises(ValueError):
        pool.table(["c"], 1)


def test_no_page_is_ever_shared():
    # random admissions and releases: every page is held by at most one
    # sequence, and held + free always covers the pool exactly
    rng = np.random.default_rng(3)
    pool = PagePool(64, 32)
    live = {}
    for i in range(2000):
        if live and (rng.random() < 0.4 or not pool.can_admit(64)):
            s = list(live)[rng.integers(len(live))]
            if rng.random() < 0.5:
                pool.release(s)
                live.pop(s)
            else:
                want = pool.length(s) + int(rng.integers(1, 80))
                if pool.pages_for(want) - len(pool.pages(s)) <= pool.free_pages:
                    pool.reserve(s, want)
        else:
            n = int(rng.integers(1, 200))
            if pool.can_admit(n):
                pool.admit(i, n)
                live[i] = True
        held = [p for s in live for p in pool.pages(s)]
        assert len(held) == len(set(held))
        assert len(held) + pool.free_pages == 64
        for s in live:
            assert len(pool.pages(s)) == pool.pages_for(pool.length(s))


def test_bad_pool_shapes():
    for args in ((0, 64), (4, 48), (4, 16)):
        with pytest.raises(ValueError):
            PagePool(*args)
