"""Several steps of a small serving loop through the library, against the
oracle at every step.

The pages' block manager gives each sequence blocks as its context grows
(a new block when the last one is full) and lets sequences share blocks by
reference, copying a shared block before anyone writes into it
(copy-on-write).  Here the library's own block pool plays that part:
prompts are written with paged_kv_write and prefilled as one chunk each
(paged_attention_prefill), then six fused decode steps follow
(paged_attention_decode_append), each sequence taking a new block when
its last one is full; at step 2 sequence 0 forks (a second sequence holds
all its blocks by reference), so the next append of either copies their
shared, partly filled last block first (pool copy-on-write plus
paged_copy_blocks); at step 3 sequence 3 is preempted (its blocks swapped
out to a pinned host pool with paged_swap_blocks and released to the
pool, where other sequences may take them) and at step 5 it resumes in
freshly allocated blocks (swapped back in).  After every step both caches equal the oracle's bit
for bit, and every output row is within |gpu - oracle| <= 2e-3 + 1e-2 *
|oracle| of the oracle's attention over the same block tables.  Run over
16-bit caches and over E4M3 caches (quantising writes, the E4M3 prefill
and decode).
"""
import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL, RTOL = 2e-3, 1e-2
HKV, HQ, D, BS, NB, MAXB = 4, 16, 128, 16, 160, 24
DT, TDT = W.BF16, torch.bfloat16
KS, VS = 0.02, 0.03


def say(msg):
    print(msg, flush=True)


def dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(TDT)


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got_bits, ref, what):
    err = np.abs(f64(got_bits) - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    say(f"  {what} max_abs={err.max():.3e} n={ref.size}")
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, worst {err[bad].max():.3e}"


def table_array(tables):
    bt = np.zeros((len(tables), MAXB), np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    return bt


def cache_bits(t):
    return t.cpu().numpy() if t.dtype == torch.uint8 else host_bits(t)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
def test_serving_loop_with_fork_and_copy_on_write(fp8):
    g = np.random.default_rng(51)
    pool = B.BlockPool(NB, order=g.permutation(NB))
    lens = [int(x) for x in g.integers(5, 120, size=6)]
    lens[0] = 37  # the sequence that forks: two full blocks and 5 tokens
    tables = [[pool.alloc() for _ in range((L + BS - 1) // BS)] for L in lens]
    assert all(b >= 0 for t in tables for b in t)
    scale = 1.0 / np.sqrt(D)

    # caches: NaN in every slot, on the device and in the oracle
    if fp8:
        kh = np.full((NB, HKV, BS, D), W.FP8_NAN, np.uint8)
        vh = np.full((NB, HKV, BS // 4, D, 4), W.FP8_NAN, np.uint8)
        kc, vc = torch.from_numpy(kh).to(DEV), torch.from_numpy(vh).to(DEV)
    else:
        kh = np.full((NB, HKV, BS, D), W.NAN_BITS[DT], np.uint16)
        vh = np.full((NB, HKV, BS // 4, D, 4), W.NAN_BITS[DT], np.uint16)
        kc, vc = dev_bits(kh), dev_bits(vh)

    def write(k, v, sl):  # the same tokens into both sides
        if fp8:
            oracle.kv_write_fp8(k, v, sl, kh, vh, BS, DT, KS, VS)
            B.paged_kv_write_fp8(dev_bits(k), dev_bits(v), torch.from_numpy(sl).to(DEV), kc, vc,
                                 KS, VS)
        else:
            oracle.kv_write(k, v, sl, kh, vh, BS)
            B.paged_kv_write(dev_bits(k), dev_bits(v), torch.from_numpy(sl).to(DEV), kc, vc)

    def attend(q, bt, cl):
        if fp8:
            return oracle.decode_fp8(q, kh, vh, bt, cl, scale, BS, DT, KS, VS)
        return oracle.decode(q, kh, vh, bt, cl, scale, BS, DT)

    fs = dict(k_scale=KS, v_scale=VS) if fp8 else {}
    # pinned host pool for swapped-out blocks, and the oracle's copy of it
    NH = 16
    hdt, ndt = (torch.uint8, np.uint8) if fp8 else (TDT, np.uint16)
    hk_t = torch.zeros((NH, HKV, BS, D), dtype=hdt).pin_memory()
    hv_t = torch.zeros((NH, HKV, BS // 4, D, 4), dtype=hdt).pin_memory()
    hkh = np.zeros((NH, HKV, BS, D), ndt)
    hvh = np.zeros((NH, HKV, BS // 4, D, 4), ndt)

    # prompts: written, then prefilled as one chunk per sequence
    slots = np.array([tables[s][p // BS] * BS + p % BS for s, L in enumerate(lens)
                      for p in range(L)], np.int64)
    pk = W.normal_bits(g, (slots.size, HKV, D), DT)
    pv = W.normal_bits(g, (slots.size, HKV, D), DT)
    write(pk, pv, slots)
    bt = table_array(tables)
    cl = np.array(lens, np.int32)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qp = W.normal_bits(g, (int(qs[-1]), HQ, D), DT)
    outp = torch.empty((int(qs[-1]), HQ, D), dtype=TDT, device=DEV)
    say(f"prefill of the prompts, fp8={fp8}")
    pargs = (outp, dev_bits(qp), kc, vc, torch.from_numpy(bt).to(DEV),
             torch.from_numpy(cl).to(DEV), torch.from_numpy(qs).to(DEV), scale)
    if fp8:
        B.paged_attention_prefill_fp8(*pargs, KS, VS, BS, HKV, max(lens))
        ref = oracle.prefill_fp8(qp, kh, vh, bt, cl, qs, scale, BS, DT, KS, VS)
    else:
        B.paged_attention_prefill(*pargs, BS, HKV, max(lens))
        ref = oracle.prefill(qp, kh, vh, bt, cl, qs, scale, BS, DT)
    torch.cuda.synchronize()
    check_close(host_bits(outp), ref, "prefill")

    active = [True] * len(lens)
    for step in range(6):
        if step == 2:  # sequence 0 forks: the new sequence holds its blocks by reference
            for b in tables[0]:
                pool.incref(b)
            tables.append(list(tables[0]))
            lens.append(lens[0])
            active.append(True)
        if step == 3:  # sequence 3 is preempted: its blocks go to the host pool
            sp = np.array([(b, i) for i, b in enumerate(tables[3])], np.int64)
            oracle.swap_blocks(sp, hkh, hvh, kh, vh, BS)
            B.paged_swap_blocks(torch.from_numpy(sp).pin_memory(), hk_t, hv_t, kc, vc)
            for b in tables[3]:
                pool.decref(b)
            active[3] = False
        if step == 5:  # and resumes in fresh blocks
            fresh = [pool.alloc() for _ in tables[3]]
            assert all(b >= 0 for b in fresh)
            sp = np.array([(i, b) for i, b in enumerate(fresh)], np.int64)
            oracle.swap_blocks(sp, kh, vh, hkh, hvh, BS)
            B.paged_swap_blocks(torch.from_numpy(sp).pin_memory(), kc, vc, hk_t, hv_t)
            tables[3] = fresh
            active[3] = True
        run = [s for s in range(len(lens)) if active[s]]
        # position L of each sequence takes the new token: a new block when the
        # last one is full, else the last block, copied first if it is shared
        pairs, new_slots = [], []
        for s in run:
            L = lens[s]
            if L % BS == 0:
                b = pool.alloc()
                assert b >= 0
                tables[s].append(b)
            else:
                dst, copy = pool.cow(tables[s][-1])
                if copy:
                    pairs.append((tables[s][-1], dst))
                tables[s][-1] = dst
            new_slots.append(tables[s][L // BS] * BS + L % BS)
            lens[s] = L + 1
        if step == 2:
            assert len(pairs) == 1, "the fork's shared last block is copied once"
        if pairs:
            pa = np.array(pairs, np.int64)
            oracle.copy_blocks(pa, kh, vh, BS)
            B.paged_copy_blocks(torch.from_numpy(pa).to(DEV), kc, vc)
        bt = table_array([tables[s] for s in run])
        cl = np.array([lens[s] for s in run], np.int32)
        n = len(run)
        q = W.normal_bits(g, (n, HQ, D), DT)
        kn = W.normal_bits(g, (n, HKV, D), DT)
        vn = W.normal_bits(g, (n, HKV, D), DT)
        out = torch.empty((n, HQ, D), dtype=TDT, device=DEV)
        say(f"decode step {step}: sequences {run}, lengths {cl.tolist()}")
        B.paged_attention_decode_append(out, dev_bits(q), dev_bits(kn), dev_bits(vn), kc, vc,
                                        torch.from_numpy(bt).to(DEV),
                                        torch.from_numpy(cl).to(DEV), scale, BS, HKV, **fs)
        torch.cuda.synchronize()
        if fp8:
            oracle.kv_write_fp8(kn, vn, np.array(new_slots, np.int64), kh, vh, BS, DT, KS, VS)
        else:
            oracle.kv_write(kn, vn, np.array(new_slots, np.int64), kh, vh, BS)
        assert np.array_equal(cache_bits(kc), kh), f"K cache, step {step}"
        assert np.array_equal(cache_bits(vc), vh), f"V cache, step {step}"
        check_close(host_bits(out), attend(q, bt, cl), f"step {step}")

    # the fork and its source still share their two full blocks; every other
    # block has one holder
    assert tables[0][:2] == tables[-1][:2]
    assert all(pool.refcount(b) == 2 for b in tables[0][:2])
    held = {b for t in tables for b in t}
    assert all(pool.refcount(b) == 1 for b in held - set(tables[0][:2]))
    assert pool.num_free == NB - len(held)
    pool.close()
