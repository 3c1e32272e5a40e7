"""The library's reference-counted block pool and the block-copy ABI on the
CPU (no GPU call): the pool against the test harness's own block manager
under random operation sequences, its copy-on-write decision, misuse,
thread safety, and the host-side rejections of paged_copy_blocks and
paged_validate_copy_pairs."""
import ctypes
import os
import re
import threading

import numpy as np
import pytest
import torch  # noqa: F401  (the binding binds to torch's HIP runtime)

from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000


def test_exports_every_declared_symbol():
    text = open(os.path.join(ROOT, "include", "paged_blocks.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))
    assert {"pa_pool_create", "pa_pool_destroy", "pa_pool_alloc", "pa_pool_incref",
            "pa_pool_decref", "pa_pool_refcount", "pa_pool_cow", "pa_pool_num_free",
            "pa_pool_num_blocks", "paged_copy_blocks", "paged_validate_copy_pairs"} <= names
    lib = B.load()
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("seed", range(6))
def test_pool_matches_harness_allocator(seed):
    """Same ids handed out and the same counts as the harness's Python
    block manager (a stack over a permutation) under random alloc / share /
    release / copy-on-write sequences."""
    g = np.random.default_rng(seed)
    nb = int(g.integers(1, 60))
    order = g.permutation(nb)
    pool = B.BlockPool(nb, order)
    ref = W.BlockAllocator(order)
    live = []
    for _ in range(600):
        op = g.integers(0, 4)
        if op == 0:
            got = pool.alloc()
            if ref.free:
                assert got == ref.allocate()
                live.append(got)
            else:
                assert got == -1
        elif op == 1 and live:
            b = live[int(g.integers(len(live)))]
            pool.incref(b)
            ref.share(b)
            live.append(b)
        elif op == 2 and live:
            b = live.pop(int(g.integers(len(live))))
            pool.decref(b)
            ref.release(b)
        elif op == 3 and live:
            i = int(g.integers(len(live)))
            b = live[i]
            if ref.refcount[b] > 1 and not ref.free:
                with pytest.raises(Exception):
                    pool.cow(b)
                continue
            dst, copy = pool.cow(b)
            if ref.refcount[b] > 1:  # the model: fresh block, one share fewer
                assert copy and dst == ref.allocate()
                ref.release(b)
                live[i] = dst
            else:
                assert not copy and dst == b
        assert pool.num_free == len(ref.free)
        for b in range(nb):
            assert pool.refcount(b) == ref.refcount.get(b, 0)
    pool.close()


def test_pool_misuse_changes_nothing():
    pool = B.BlockPool(4)
    b = pool.alloc()
    for bad in (-1, 4, 99):
        with pytest.raises(Exception):
            pool.incref(bad)
        with pytest.raises(Exception):
            pool.decref(bad)
        with pytest.raises(Exception):
            pool.cow(bad)
        assert pool.refcount(bad) == -1
    free_block = 3 if b != 3 else 2
    with pytest.raises(Exception):
        pool.incref(free_block)     # a free block has no sharer to add to
    with pytest.raises(Exception):
        pool.decref(free_block)
    assert pool.num_free == 3 and pool.refcount(b) == 1
    pool.decref(b)
    with pytest.raises(Exception):
        pool.decref(b)              # already back in the pool
    assert pool.num_free == 4


def test_pool_create_rejects_bad_order():
    for order in ([0, 0, 1], [0, 1, 3], [-1, 0, 1]):
        with pytest.raises(ValueError):
            B.BlockPool(3, order)
    with pytest.raises(ValueError):
        B.BlockPool(0)


def test_cow_when_exhausted():
    pool = B.BlockPool(1)
    b = pool.alloc()
    pool.incref(b)
    with pytest.raises(Exception):
        pool.cow(b)                 # shared, and no block left for the copy
    assert pool.refcount(b) == 2 and pool.num_free == 0


def test_pool_threads_hand_out_distinct_blocks():
    pool = B.BlockPool(8000)
    got = [[] for _ in range(8)]

    def worker(i):
        for _ in range(1000):
            got[i].append(pool.alloc())

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    flat = sorted(x for part in got for x in part)
    assert flat == list(range(8000)) and pool.num_free == 0


def _copy(**kw):
    a = dict(kc=FAKE, vc=FAKE, pairs=FAKE, n=4, hkv=8, d=128, bs=16, nb=100, eb=2, stream=None)
    a.update(kw)
    return B.load().paged_copy_blocks(a["kc"], a["vc"], a["pairs"], a["n"], a["hkv"], a["d"],
                                      a["bs"], a["nb"], a["eb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(eb=4), -2), (dict(d=96), -3), (dict(bs=12), -3), (dict(nb=0), -3), (dict(n=-1), -3),
    (dict(hkv=0), -3), (dict(kc=None), -1), (dict(pairs=None), -1),
    (dict(kc=FAKE + 8), -7), (dict(pairs=FAKE + 4), -7),
])
def test_copy_rejects_before_launch(kw, code):
    assert _copy(**kw) == code


def test_copy_zero_pairs_is_noop():
    assert _copy(n=0, kc=None, vc=None, pairs=None) == 0


@pytest.mark.parametrize("pairs,code", [
    ([(0, 1), (2, 3), (-1, 5), (4, -1)], 0),
    ([(0, 1), (0, 2), (0, 3)], 0),         # one source, many copies (a fork)
    ([(0, 1), (2, 1)], -6),                # destination twice
    ([(0, 1), (1, 2)], -6),                # destination also a source
    ([(0, 10)], -6), ([(10, 0)], -6),      # past the pool
    ([], 0),
])
def test_validate_copy_pairs(pairs, code):
    assert B.validate_copy_pairs(np.array(pairs, np.int64).reshape(-1, 2), 10) == code


def _swap(**kw):
    a = dict(dk=FAKE, dv=FAKE, dn=100, sk=FAKE, sv=FAKE, sn=50, pairs=FAKE, n=4, hkv=8, d=128,
             bs=16, eb=2, stream=None)
    a.update(kw)
    return B.load().paged_swap_blocks(a["dk"], a["dv"], a["dn"], a["sk"], a["sv"], a["sn"],
                                      a["pairs"], a["n"], a["hkv"], a["d"], a["bs"], a["eb"],
                                      a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(eb=3), -2), (dict(d=32), -3), (dict(bs=64), -3), (dict(dn=0), -3), (dict(sn=-5), -3),
    (dict(n=-2), -3), (dict(sk=None), -1), (dict(dv=None), -1), (dict(pairs=None), -1),
    (dict(sv=FAKE + 4), -7), (dict(dk=FAKE + 2), -7), (dict(pairs=FAKE + 2), -7),
])
def test_swap_rejects_before_launch(kw, code):
    assert _swap(**kw) == code


def test_swap_zero_pairs_is_noop():
    assert _swap(n=0, dk=None, dv=None, sk=None, sv=None, pairs=None) == 0


@pytest.mark.parametrize("pairs,code", [
    ([(0, 1), (2, 3), (-1, 5), (4, -1)], 0),
    ([(0, 1), (0, 2)], 0),                 # one device block to two host slots
    ([(0, 1), (1, 0)], 0),                 # distinct pools: a source may share an id with a dst
    ([(0, 1), (2, 1)], -6),
    ([(0, 20)], -6), ([(10, 0)], -6),      # past the destination / source pool
])
def test_validate_swap_pairs(pairs, code):
    assert B.validate_swap_pairs(np.array(pairs, np.int64).reshape(-1, 2), 10, 20) == code
