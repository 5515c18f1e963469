"""The host page allocator: the oracle model pinned to the page's admission figures and to
invariants, and the library's allocator equal to the model, state for state, over seeded random
operation sequences (bit-exact: page IDs, free-list order, reference counts, reservations)."""
import random

import pytest

from oracle import pages as model
from compressed_kv_attention_kvexec_amd.pages import PageAllocator

P = 256
POOL = 896  # 229,376 positions in 256-position pages


def test_model_admission_matches_the_page_figures():
    # one request of 196,608 prompt + 16,384 output tokens reserves (196,608 + 8,192) / 256 pages
    assert model.admission_need(196608, 16384, P) == 800
    assert model.admission_need(196608, 16384, P) * P <= 212992
    # two requests of 96K + 16K: 416 pages reserved each, 448 held each at the end, which fills the
    # 229,376-position pool exactly
    pool = model.PagePool(POOL, P)
    a = pool.admit(98304, 16384)
    b = pool.admit(98304, 16384)
    assert pool.reserved == 832
    assert pool.extend(a, 98304 + 16384) and pool.extend(b, 98304 + 16384)
    assert len(pool.free) == 0 and len(pool.table(a)) + len(pool.table(b)) == 896
    # the four-request mix (128K + 12K and three of 8K + 12K) fits: 544 + 3 x 64 reserved, 800 held
    pool = model.PagePool(POOL, P)
    ids = [pool.admit(131072, 12288)] + [pool.admit(8192, 12288) for _ in range(3)]
    assert pool.reserved == 544 + 3 * 64
    for rid, L in zip(ids, [143360] + [20480] * 3):
        assert pool.extend(rid, L)
    assert sum(len(pool.table(r)) for r in ids) * P == 204800


def test_model_reservation_and_deferred_release():
    pool = model.PagePool(10, 4)
    a = pool.admit(8, 8)            # need ceil(16 / 4) = 4
    assert pool.admit(20, 8) is None  # 4 + 7 > 10
    b = pool.admit(12, 4)           # need 4 -> 8 reserved
    assert pool.reserved == 8
    assert pool.extend(a, 8) and pool.table(a) == [0, 1]
    c = pool.admit(8, 0, prefix_pages=[0])  # shares a's first page
    assert pool.refcount[0] == 2 and pool.table(c) == [0]
    assert pool.extend(c, 8) and pool.table(c) == [0, 2]
    pool.finish(a)
    assert pool.refcount[0] == 2 and 0 not in pool.free  # nothing returns before the boundary
    pool.boundary()
    assert pool.refcount[0] == 1 and list(pool.free)[-1] == 1  # page 1 back, page 0 still held by c
    pool.finish(c)
    pool.boundary()
    assert list(pool.free)[-2:] == [0, 2]  # c's table order
    assert pool.extend(b, 16) and pool.table(b) == [3, 4, 5, 6]


def _invariants(pool):
    held = {}
    for r in pool.requests:
        if r[2]:
            for p in r[1]:
                held[p] = held.get(p, 0) + 1
    assert all(pool.refcount[p] == held.get(p, 0) for p in range(pool.num_pages))
    assert sorted(pool.free) == sorted(p for p in range(pool.num_pages) if p not in held)
    assert pool.reserved == sum(r[0] for r in pool.requests if r[2])


def _random_ops(seed, n_ops, num_pages, page):
    rng = random.Random(seed)
    ops, live = [], []
    for _ in range(n_ops):
        x = rng.random()
        if x < 0.3 or not live:
            ops.append(("admit", rng.randrange(0, 6 * page), rng.randrange(0, 4 * page), rng.random()))
        elif x < 0.65:
            ops.append(("extend", rng.random(), rng.randrange(0, 10 * page)))
        elif x < 0.85:
            ops.append(("finish", rng.random()))
        else:
            ops.append(("boundary",))
    return ops


@pytest.mark.parametrize("seed,num_pages,page", [(1, 40, 4), (2, 16, 1), (3, 200, 32), (4, 7, 3)])
def test_library_allocator_equals_model(seed, num_pages, page):
    ref = model.PagePool(num_pages, page)
    lib = PageAllocator(num_pages, page)
    live = []  # live, not departing request ids (same in both)
    for op in _random_ops(seed, 1500, num_pages, page):
        if op[0] == "admit":
            _, prompt, out, u = op
            prefix = []
            if live and u < 0.5:  # share whole pages of a live request's table
                donor = live[int(u * 2 * len(live)) % len(live)]
                full = min(len(ref.table(donor)), prompt // page)
                prefix = ref.table(donor)[:full]
            r1, r2 = ref.admit(prompt, out, prefix), lib.admit(prompt, out, prefix)
            assert r1 == r2
            if r1 is not None:
                live.append(r1)
        elif op[0] == "extend":
            rid = live[int(op[1] * len(live))]
            assert ref.extend(rid, op[2]) == lib.extend(rid, op[2])
        elif op[0] == "finish":
            rid = live.pop(int(op[1] * len(live)))
            ref.finish(rid)
            lib.finish(rid)
        else:
            ref.boundary()
            lib.boundary()
        _invariants(ref)
        assert lib.free_list() == list(ref.free)
        assert lib.reserved() == ref.reserved
        assert [lib.refcount(p) for p in range(num_pages)] == ref.refcount
        for rid in live:
            assert lib.table(rid) == ref.table(rid)
    lib.close()


def test_library_rejects_bad_arguments():
    from compressed_kv_attention_kvexec_amd import _binding as B
    import ctypes
    lib = B.load_library()
    h = ctypes.c_void_p()
    assert lib.tq4_pages_create(0, 4, ctypes.byref(h)) == 2
    assert lib.tq4_pages_create(4, 4, None) == 1
    assert lib.tq4_pages_admission_need(-1, 0, 256) == -1
    assert lib.tq4_pages_admission_need(100, 20000, 256) == (100 + 8192 + 255) // 256
    a = PageAllocator(4, 4)
    with pytest.raises(B.Tq4Error):
        a.admit(4, 0, prefix_pages=[2])   # page 2 is not held
    rid = a.admit(4, 0)
    assert a.extend(rid, 4)
    with pytest.raises(B.Tq4Error):
        a.admit(3, 0, prefix_pages=[0])   # a whole page longer than the prompt
    with pytest.raises(B.Tq4Error):
        a.extend(99, 4)
    a.finish(rid)
    with pytest.raises(B.Tq4Error):
        a.finish(rid)                     # already departing
    a.boundary()
    with pytest.raises(B.Tq4Error):
        a.table(rid)                      # dead handle
    a.close()
