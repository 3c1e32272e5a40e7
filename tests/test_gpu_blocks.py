"""GPU parity of paged_copy_blocks (copy-on-write block copy) through the C
ABI, and of a copy-on-write decode flow driven by the library's block pool.

* paged_copy_blocks: bit-exact against oracle_copy_blocks over both whole
  caches, for 16-bit and E4M3 (1-byte) caches, every head_dim and block
  size, fan-out from one source, skipped pairs (negative ids, ids past the
  pool), and a batch of several thousand pairs;
* copy-on-write flow: forks of a prompt whose last block is partly filled,
  with the library's pool deciding each copy (pa_pool_cow) and the device
  copying and appending, leave caches and tables bit-identical to the same
  flow on the oracle, and decode meets |gpu - oracle| <= 2e-3 +
  1e-2 * |oracle| against the oracle over the tokens stored privately.
"""
import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W
from test_oracle_blocks import fork_with_cow, private_layout, rand_caches

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)


def to_dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def to_host(t, like):
    a = t.cpu().numpy()
    return a.view(np.uint16) if like.dtype == np.uint16 else a


def run_copy(k, v, pairs):
    kd, vd = to_dev(k), to_dev(v)
    B.paged_copy_blocks(torch.from_numpy(np.asarray(pairs, np.int64).reshape(-1, 2)).to(DEV),
                        kd, vd)
    torch.cuda.synchronize()
    return to_host(kd, k), to_host(vd, v)


@pytest.mark.parametrize("itemsize", [2, 1])
@pytest.mark.parametrize("hkv,bs,d", [(1, 8, 64), (2, 16, 128), (8, 32, 64), (8, 16, 128),
                                      (3, 32, 128)])
def test_copy_bit_exact(itemsize, hkv, bs, d):
    g = np.random.default_rng(500 + hkv * 10 + bs + d + itemsize)
    nb = 64
    k, v = rand_caches(g, nb, hkv, bs, d, itemsize)
    ids = g.permutation(nb)
    pairs = [(int(ids[i % 7]), int(ids[10 + i])) for i in range(30)]  # fan-out
    pairs += [(-1, int(ids[50])), (int(ids[51]), -1), (nb + 3, int(ids[52])),
              (int(ids[53]), nb)]                                        # skipped on the device
    say(f"copy hkv={hkv} bs={bs} d={d} itemsize={itemsize}")
    gk, gv = run_copy(k, v, pairs)
    ok_pairs = [(s, t) for s, t in pairs if 0 <= s < nb and 0 <= t < nb]
    ek, ev = k.copy(), v.copy()
    oracle.copy_blocks(np.array(ok_pairs), ek, ev, bs)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


def test_copy_large_batch():
    """Several thousand pairs (more than one launch's worth of small runs)."""
    g = np.random.default_rng(9)
    nb, hkv, bs, d = 12000, 2, 16, 64
    k, v = rand_caches(g, nb, hkv, bs, d, 2)
    ids = g.permutation(nb)
    pairs = np.stack([ids[:5000], ids[5000:10000]], axis=1)
    say("copy 5000 pairs")
    gk, gv = run_copy(k, v, pairs)
    ek, ev = k.copy(), v.copy()
    oracle.copy_blocks(pairs, ek, ev, bs)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_cow_flow_on_device(bs):
    hkv, d, G, prompt, suffix = 2, 64, 4, 45, [1, 3, bs, 2 * bs + 5]
    ok, ov, obt, lens, logical, _, order = fork_with_cow(prompt, suffix, bs, hkv, d,
                                                         seed=60 + bs)
    nb = ok.shape[0]
    pool = B.BlockPool(nb, order)
    nan = int(np.array([W.NAN_BITS[W.BF16]], np.uint16).view(np.int16)[0])
    kc = torch.full((nb, hkv, bs, d), nan, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    vc = torch.full((nb, hkv, bs // 4, d, 4), nan, dtype=torch.int16, device=DEV).view(torch.bfloat16)

    def put(kk, vv, slot):
        B.paged_kv_write(torch.from_numpy(kk.view(np.int16)).to(DEV).view(torch.bfloat16),
                         torch.from_numpy(vv.view(np.int16)).to(DEV).view(torch.bfloat16),
                         torch.tensor([slot], dtype=torch.int64, device=DEV), kc, vc)

    pk, pv = logical[0][0][:prompt], logical[0][1][:prompt]
    root = []
    for t in range(prompt):
        if t % bs == 0:
            root.append(pool.alloc())
        put(pk[t:t + 1], pv[t:t + 1], root[t // bs] * bs + t % bs)
    tables = []
    copies = 0
    for s, n_own in enumerate(suffix):
        table = list(root)
        for b in root:
            pool.incref(b)
        n = prompt
        sk, sv = logical[s][0][prompt:], logical[s][1][prompt:]
        for i in range(n_own):
            if n % bs == 0:
                table.append(pool.alloc())
            else:
                dst, copy = pool.cow(table[n // bs])
                if copy:
                    B.paged_copy_blocks(torch.tensor([[table[n // bs], dst]], dtype=torch.int64,
                                                     device=DEV), kc, vc)
                    copies += 1
                    table[n // bs] = dst
            put(sk[i:i + 1], sv[i:i + 1], table[n // bs] * bs + n % bs)
            n += 1
        tables.append(table)
    for b in root:
        pool.decref(b)
    torch.cuda.synchronize()
    say(f"cow flow bs={bs}: {copies} block copies")
    assert copies == (len(suffix) if prompt % bs else 0)
    bt = np.zeros_like(obt)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    assert np.array_equal(bt, obt)
    hk = kc.view(torch.int16).cpu().numpy().view(np.uint16)
    hv = vc.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(hk, ok) and np.array_equal(hv, ov)
    # decode over the copy-on-write layout against the private-copy oracle
    g = np.random.default_rng(7)
    q = W.normal_bits(g, (len(suffix), hkv * G, d), W.BF16)
    qd = torch.from_numpy(q.view(np.int16)).to(DEV).view(torch.bfloat16)
    out = torch.empty_like(qd)
    B.paged_attention_decode(out, qd, kc, vc, torch.from_numpy(bt).to(DEV),
                             torch.from_numpy(lens).to(DEV), 0.125, bs, hkv)
    torch.cuda.synchronize()
    pkc, pvc, pbt = private_layout(logical, bs, hkv, d)
    ref = oracle.decode(q, pkc, pvc, pbt, lens, 0.125, bs, W.BF16)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref))


# ---- swap between the device caches and a pinned host pool ---------------------

def pinned(a):
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.pin_memory()


@pytest.mark.parametrize("itemsize", [2, 1])
@pytest.mark.parametrize("hkv,bs,d", [(2, 16, 128), (8, 8, 64), (1, 32, 128)])
def test_swap_out_and_in_bit_exact(itemsize, hkv, bs, d):
    g = np.random.default_rng(800 + hkv + bs + d + itemsize)
    nd, nh = 96, 40
    dk, dv = rand_caches(g, nd, hkv, bs, d, itemsize)
    hk, hv = rand_caches(g, nh, hkv, bs, d, itemsize)
    dkt, dvt = to_dev(dk), to_dev(dv)
    hkt, hvt = pinned(hk), pinned(hv)
    ids = g.permutation(nd)
    out_pairs = np.stack([ids[:30], g.permutation(nh)[:30]], 1)
    out_pairs = np.concatenate([out_pairs, [[-1, 35], [3, -1], [nd + 1, 36]]])
    say(f"swap out hkv={hkv} bs={bs} d={d} itemsize={itemsize}")
    B.paged_swap_blocks(torch.from_numpy(out_pairs).to(DEV), hkt, hvt, dkt, dvt)
    torch.cuda.synchronize()
    ek, ev = hk.copy(), hv.copy()
    ok_pairs = [(s, t) for s, t in out_pairs if 0 <= s < nd and 0 <= t < nh]
    oracle.swap_blocks(np.array(ok_pairs), ek, ev, dk, dv, bs)
    assert np.array_equal(to_host(hkt, hk), ek) and np.array_equal(to_host(hvt, hv), ev)
    in_pairs = np.stack([np.arange(nh), ids[40:40 + nh]], 1)          # pairs in pinned memory
    say("swap in")
    B.paged_swap_blocks(torch.from_numpy(in_pairs).pin_memory(), dkt, dvt, hkt, hvt,
                        stream_device=torch.device(DEV))
    torch.cuda.synchronize()
    fk, fv = dk.copy(), dv.copy()
    oracle.swap_blocks(in_pairs, fk, fv, ek, ev, bs)
    assert np.array_equal(to_host(dkt, dk), fk) and np.array_equal(to_host(dvt, dv), fv)


def test_preempt_and_resume_on_device():
    """Swap a sequence out to pinned host memory, overwrite its device
    blocks, swap it back into other blocks and rewrite its table: decode is
    bit-identical to the decode before preemption."""
    w = W.build("swapg", [300, 77, 512, 1000], num_heads=16, num_kv_heads=2, head_dim=128,
                block_size=16, dtype=W.BF16, seed=13, pool=200, max_blocks_per_seq=70)
    ksh, vsh = w.cache_shapes()
    kc = torch.zeros(ksh, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros(vsh, dtype=torch.bfloat16, device=DEV)
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        B.paged_kv_write(torch.from_numpy(k.view(np.int16)).to(DEV).view(torch.bfloat16),
                         torch.from_numpy(v.view(np.int16)).to(DEV).view(torch.bfloat16),
                         torch.from_numpy(s).to(DEV), kc, vc)
    q = torch.from_numpy(w.q.view(np.int16)).to(DEV).view(torch.bfloat16)
    cl = torch.from_numpy(w.context_lens).to(DEV)

    def decode(bt):
        out = torch.empty_like(q)
        B.paged_attention_decode(out, q, kc, vc, torch.from_numpy(bt).to(DEV), cl, w.scale,
                                 16, 2)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy()

    before = decode(w.block_tables)
    seq = 3
    used = int(np.ceil(w.context_lens[seq] / 16))
    blocks = w.block_tables[seq, :used].copy()
    hk = torch.empty((used,) + ksh[1:], dtype=torch.bfloat16).pin_memory()
    hv = torch.empty((used,) + vsh[1:], dtype=torch.bfloat16).pin_memory()
    say(f"preempt seq {seq}: {used} blocks out")
    B.paged_swap_blocks(torch.from_numpy(np.stack([blocks, np.arange(used)], 1)).to(DEV),
                        hk, hv, kc, vc)
    kc[torch.from_numpy(blocks).to(DEV)] = float("nan")   # the blocks are reused meanwhile
    vc[torch.from_numpy(blocks).to(DEV)] = float("nan")
    in_use = set(w.block_tables.ravel().tolist())
    fresh = np.array([b for b in range(200) if b not in in_use][:used])
    B.paged_swap_blocks(torch.from_numpy(np.stack([np.arange(used), fresh], 1)).to(DEV),
                        kc, vc, hk, hv)
    bt = w.block_tables.copy()
    bt[seq, :used] = fresh
    after = decode(bt)
    assert np.array_equal(before, after)
