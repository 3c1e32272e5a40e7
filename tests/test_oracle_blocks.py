"""Pins of the oracle's block copy (copy-on-write, "vLLM framework analysis:
how PagedAttention achieves a 20x LLM inference speed-up", 2.3) against
things other than itself (no GPU):

* numpy block slicing: after the copy, block dst of each cache equals block
  src as a whole slice, and every other block is unchanged (the oracle walks
  elements through its own index arithmetic; the slice does not);
* skipped pairs (negative ids) and refused pairs (repeated destination, a
  destination that is also a source, an id past the pool) leave the caches
  untouched;
* swap (block moves between a device pool and a host pool): against numpy
  slices both ways, refused pairs, and a preempt/resume round trip whose
  decode is bit-identical to the one before preemption;
* copy-on-write end to end: sequences forked from a prompt whose last block
  is only partly filled share every prompt block; each fork's first append
  copies the shared partial block (a reference model of the decision in the
  test: share count > 1 -> fresh block + copy) and then writes; the oracle
  decode over that layout equals, bit for bit, the oracle decode over the
  same logical tokens stored privately per sequence.
"""
import numpy as np
import pytest

import oracle
from pagedattention_kv_cache_paged_amd import workloads as W


def rand_caches(g, nb, hkv, bs, d, itemsize):
    dt = np.uint16 if itemsize == 2 else np.uint8
    hi = 1 << (8 * itemsize)
    k = g.integers(0, hi, size=(nb, hkv, bs, d), dtype=np.int64).astype(dt)
    v = g.integers(0, hi, size=(nb, hkv, bs // 4, d, 4), dtype=np.int64).astype(dt)
    return k, v


@pytest.mark.parametrize("itemsize", [2, 1])
@pytest.mark.parametrize("hkv,bs,d", [(1, 8, 64), (2, 16, 128), (8, 32, 64)])
def test_copy_equals_block_slices(itemsize, hkv, bs, d):
    g = np.random.default_rng(hkv * 100 + bs + d + itemsize)
    nb = 40
    k, v = rand_caches(g, nb, hkv, bs, d, itemsize)
    ids = g.permutation(nb)
    srcs = ids[:10]
    dsts = ids[10:22]
    pairs = [(int(srcs[i % 10]), int(dsts[i])) for i in range(12)]  # fan-out from sources
    pairs += [(-1, int(ids[30])), (int(ids[31]), -1)]                  # skipped
    k0, v0 = k.copy(), v.copy()
    oracle.copy_blocks(np.array(pairs), k, v, bs)
    ek, ev = k0.copy(), v0.copy()
    for s_, d_ in pairs:
        if s_ >= 0 and d_ >= 0:
            ek[d_] = k0[s_]
            ev[d_] = v0[s_]
    assert np.array_equal(k, ek) and np.array_equal(v, ev)
    touched = {d_ for s_, d_ in pairs if s_ >= 0 and d_ >= 0}
    for b in range(nb):
        if b not in touched:
            assert np.array_equal(k[b], k0[b]) and np.array_equal(v[b], v0[b])


@pytest.mark.parametrize("pairs", [
    [(1, 2), (3, 2)],        # destination twice
    [(1, 2), (2, 3)],        # a destination is also a source
    [(1, 40)],               # past the pool
    [(40, 1)],
])
def test_copy_refuses_bad_pairs(pairs):
    g = np.random.default_rng(5)
    k, v = rand_caches(g, 40, 2, 16, 64, 2)
    k0, v0 = k.copy(), v.copy()
    with pytest.raises(oracle.OracleError):
        oracle.copy_blocks(np.array(pairs), k, v, 16)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)


def fork_with_cow(prompt_len, suffix_lens, bs, hkv, d, seed):
    """Oracle caches and tables of forks that share a prompt (including its
    partly filled last block) and then append their own tokens, copying a
    shared block before the first write into it.  Returns the caches,
    tables, lengths, each sequence's logical K/V, the allocator and the
    block order it handed out from."""
    g = np.random.default_rng(seed)
    B = len(suffix_lens)
    total = prompt_len + max(suffix_lens)
    nb = 2 * (B * (total // bs + 2))
    order = g.permutation(nb)
    alloc = W.BlockAllocator(order)
    kc, vc = (np.full((nb, hkv, bs, d), W.NAN_BITS[W.BF16], np.uint16),
              np.full((nb, hkv, bs // 4, d, 4), W.NAN_BITS[W.BF16], np.uint16))
    pk = W.normal_bits(g, (prompt_len, hkv, d), W.BF16)
    pv = W.normal_bits(g, (prompt_len, hkv, d), W.BF16)
    root = []
    for t in range(prompt_len):
        if t % bs == 0:
            root.append(alloc.allocate())
        slot = np.array([root[t // bs] * bs + t % bs], np.int64)
        oracle.kv_write(pk[t:t + 1], pv[t:t + 1], slot, kc, vc, bs)
    tables, logical = [], []
    for s in range(B):
        table = [alloc.share(b) for b in root]
        n = prompt_len
        sk = W.normal_bits(g, (suffix_lens[s], hkv, d), W.BF16)
        sv = W.normal_bits(g, (suffix_lens[s], hkv, d), W.BF16)
        for i in range(suffix_lens[s]):
            if n % bs == 0:
                table.append(alloc.allocate())
            else:
                last = table[n // bs]
                if alloc.refcount[last] > 1:  # shared: copy before writing
                    fresh = alloc.allocate()
                    alloc.release(last)
                    oracle.copy_blocks(np.array([[last, fresh]]), kc, vc, bs)
                    table[n // bs] = fresh
            slot = np.array([table[n // bs] * bs + n % bs], np.int64)
            oracle.kv_write(sk[i:i + 1], sv[i:i + 1], slot, kc, vc, bs)
            n += 1
        tables.append(table)
        logical.append((np.concatenate([pk, sk]), np.concatenate([pv, sv])))
    for b in root:
        alloc.release(b)
    mb = max(len(t) for t in tables)
    bt = np.zeros((B, mb), np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    lens = np.array([prompt_len + x for x in suffix_lens], np.int32)
    return kc, vc, bt, lens, logical, alloc, order


def private_layout(logical, bs, hkv, d):
    """The same logical tokens, each sequence in its own consecutive blocks."""
    B = len(logical)
    per = [int(np.ceil(len(k) / bs)) for k, _ in logical]
    nb = sum(per)
    kc = np.full((nb, hkv, bs, d), W.NAN_BITS[W.BF16], np.uint16)
    vc = np.full((nb, hkv, bs // 4, d, 4), W.NAN_BITS[W.BF16], np.uint16)
    bt = np.zeros((B, max(per)), np.int32)
    base = 0
    for s, (k, v) in enumerate(logical):
        bt[s, :per[s]] = np.arange(base, base + per[s])
        slots = base * bs + np.arange(len(k), dtype=np.int64)
        oracle.kv_write(k, v, slots, kc, vc, bs)
        base += per[s]
    return kc, vc, bt


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_cow_fork_equals_private_copies(bs):
    hkv, d, G = 2, 64, 4
    kc, vc, bt, lens, logical, alloc, _ = fork_with_cow(45, [1, 3, bs, 2 * bs + 5], bs, hkv, d,
                                                     seed=60 + bs)
    # the shared partial block was copied once per fork; full prompt blocks stay shared
    full = 45 // bs
    assert all(alloc.refcount[bt[s, i]] == 4 for s in range(4) for i in range(full))
    assert len({int(bt[s, full]) for s in range(4)}) == 4
    g = np.random.default_rng(7)
    q = W.normal_bits(g, (4, hkv * G, d), W.BF16)
    got = oracle.decode(q, kc, vc, bt, lens, 0.125, bs, W.BF16)
    pk, pv, pbt = private_layout(logical, bs, hkv, d)
    ref = oracle.decode(q, pk, pv, pbt, lens, 0.125, bs, W.BF16)
    assert np.array_equal(got, ref)


# ---- swap between two pools ---------------------------------------------------

@pytest.mark.parametrize("itemsize", [2, 1])
def test_swap_equals_block_slices(itemsize):
    g = np.random.default_rng(70 + itemsize)
    dk, dv = rand_caches(g, 50, 2, 16, 64, itemsize)   # device pool
    hk, hv = rand_caches(g, 20, 2, 16, 64, itemsize)   # host pool
    hk0, hv0 = hk.copy(), hv.copy()
    out_pairs = np.array([(5, 0), (17, 3), (49, 19), (-1, 4), (6, -1)])
    oracle.swap_blocks(out_pairs, hk, hv, dk, dv, 16)          # swap-out: device -> host
    ek, ev = hk0.copy(), hv0.copy()
    for s_, d_ in out_pairs:
        if s_ >= 0 and d_ >= 0:
            ek[d_], ev[d_] = dk[s_], dv[s_]
    assert np.array_equal(hk, ek) and np.array_equal(hv, ev)
    dk0, dv0 = dk.copy(), dv.copy()
    in_pairs = np.array([(0, 30), (3, 31), (19, 32)])
    oracle.swap_blocks(in_pairs, dk, dv, hk, hv, 16)           # swap-in: host -> device
    for (s_, _), (_, d_) in zip(out_pairs[:3], in_pairs):
        assert np.array_equal(dk[d_], dk0[s_]) and np.array_equal(dv[d_], dv0[s_])
    untouched = [b for b in range(50) if b not in (30, 31, 32)]
    assert np.array_equal(dk[untouched], dk0[untouched])


@pytest.mark.parametrize("pairs", [[(1, 2), (3, 2)], [(1, 20)], [(50, 1)]])
def test_swap_refuses_bad_pairs(pairs):
    g = np.random.default_rng(8)
    dk, dv = rand_caches(g, 50, 2, 16, 64, 2)
    hk, hv = rand_caches(g, 20, 2, 16, 64, 2)
    hk0 = hk.copy()
    with pytest.raises(oracle.OracleError):
        oracle.swap_blocks(np.array(pairs), hk, hv, dk, dv, 16)
    assert np.array_equal(hk, hk0)


def test_preempt_and_resume_decodes_the_same():
    """Swap a sequence's blocks out, reuse its device blocks for other data,
    swap it back into different blocks and point its table there: the
    oracle's decode is bit-identical to the one before preemption."""
    w = W.build("swap", [300, 77, 512], num_heads=8, num_kv_heads=2, head_dim=64,
                block_size=16, dtype=W.BF16, seed=12, pool=80, max_blocks_per_seq=40)
    kc, vc = w.nan_caches()
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        oracle.kv_write(k, v, s, kc, vc, 16)
    before = oracle.decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, 16, w.dtype)
    seq = 0
    used = int(np.ceil(w.context_lens[seq] / 16))
    blocks = w.block_tables[seq, :used].copy()
    hk = np.zeros((used, 2, 16, 64), np.uint16)
    hv = np.zeros((used, 2, 4, 64, 4), np.uint16)
    oracle.swap_blocks(np.stack([blocks, np.arange(used)], 1), hk, hv, kc, vc, 16)
    kc[blocks] = 0x7FC0                      # the freed blocks now hold something else
    vc[blocks] = 0x7FC0
    in_use = set(w.block_tables[:, :40].ravel().tolist())
    fresh = np.array([b for b in range(80) if b not in in_use][:used])
    oracle.swap_blocks(np.stack([np.arange(used), fresh], 1), kc, vc, hk, hv, 16)
    bt = w.block_tables.copy()
    bt[seq, :used] = fresh
    after = oracle.decode(w.q, kc, vc, bt, w.context_lens, w.scale, 16, w.dtype)
    assert np.array_equal(before, after)
