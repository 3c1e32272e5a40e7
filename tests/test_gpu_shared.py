"""GPU parity of the shared-prefix decode (paged_attention_decode_shared)
through the C ABI.

Every sequence's first shared_blocks table entries are one set of physical
blocks, held by reference ("vLLM framework analysis: how PagedAttention
speeds up LLM inference 20x" (intelliparadigm.com), 2.3).  The kernels
stream those blocks once per group of sequences and merge them with each
sequence's own tiles; the oracle knows nothing of this and walks each
sequence's table token by token.  Checked against the oracle, element by
element with |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| over every output row:
the prefix workload (1024 shared tokens, 128 sequences) for the decode and
the fused step, 16-bit and E4M3 caches (caches bit-exact after the fused
step); ragged shapes over head_dim, block size, GQA group (padded column
groups included), batch sizes from 1, prefixes of one tile to several
chunks, an odd number of shared blocks at block size 8, sequences with no
private token, and three splits of the private tiles.  shared_blocks = 0 is
bit-identical to paged_attention_decode.
"""
import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {W.F16: torch.float16, W.BF16: torch.bfloat16}
ATOL, RTOL = 2e-3, 1e-2
KS, VS = 0.02, 0.03


def say(msg):
    print(msg, flush=True)


def dev_bits(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(TD[dtype])


def host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got_bits, ref, dtype, what):
    err = np.abs(f64(got_bits, dtype) - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    say(f"  {what} max_abs={err.max():.3e} n={ref.size}")
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, worst {err[bad].max():.3e}"


def caches(w, fp8, with_new):
    """Device caches (NaN everywhere else) holding the history, and the new
    tokens too when with_new."""
    ks, vs = w.cache_shapes()
    if fp8:
        kc = torch.full(ks, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        vc = torch.full(vs, W.FP8_NAN, dtype=torch.uint8, device=DEV)
    else:
        nan = int(np.array([W.NAN_BITS[w.dtype]], np.uint16).view(np.int16)[0])
        kc = torch.full(ks, nan, dtype=torch.int16, device=DEV).view(TD[w.dtype])
        vc = torch.full(vs, nan, dtype=torch.int16, device=DEV).view(TD[w.dtype])
    for which in (("hist", "new") if with_new else ("hist",)):
        k, v, s = w.write_batch(which)
        if s.size == 0:
            continue
        args = (dev_bits(k, w.dtype), dev_bits(v, w.dtype), torch.from_numpy(s).to(DEV), kc, vc)
        if fp8:
            B.paged_kv_write_fp8(*args, KS, VS)
        else:
            B.paged_kv_write(*args)
    return kc, vc


def oracle_caches(w, fp8):
    kc, vc = w.nan_caches_fp8() if fp8 else w.nan_caches()
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        if fp8:
            oracle.kv_write_fp8(k, v, s, kc, vc, w.block_size, w.dtype, KS, VS)
        else:
            oracle.kv_write(k, v, s, kc, vc, w.block_size)
    return kc, vc


def oracle_rows(w, kc, vc, fp8, context_lens=None):
    rows = oracle.all_rows(w.num_seqs, w.num_heads)
    cl = w.context_lens if context_lens is None else context_lens
    if fp8:
        ref = oracle.decode_fp8_rows(rows, w.q, kc, vc, w.block_tables, cl, w.scale,
                                     w.block_size, w.dtype, KS, VS,
                                     threads=oracle.host_threads())
    else:
        ref = oracle.decode_rows(rows, w.q, kc, vc, w.block_tables, cl, w.scale, w.block_size,
                                 w.dtype, threads=oracle.host_threads())
    return ref.reshape(w.num_seqs, w.num_heads, w.head_dim)


def run_shared(w, shared_blocks, fp8=False, append=False, cl=None, pt=0):
    kc, vc = caches(w, fp8, with_new=not append)
    q = dev_bits(w.q, w.dtype)
    out = torch.full_like(q, float("nan"))
    kw = {}
    if append:
        kn, vn, _ = w.write_batch("new")
        kw = dict(k_new=dev_bits(kn, w.dtype), v_new=dev_bits(vn, w.dtype))
    if fp8:
        kw.update(k_scale=KS, v_scale=VS)
    lens = w.context_lens if cl is None else cl
    B.paged_attention_decode_shared(out, q, kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                                    torch.from_numpy(lens).to(DEV), w.scale, w.block_size,
                                    w.num_kv_heads, shared_blocks, partition_tokens=pt, **kw)
    torch.cuda.synchronize()
    if fp8:
        return host_bits(out), kc.cpu().numpy(), vc.cpu().numpy()
    return host_bits(out), host_bits(kc), host_bits(vc)


# ---- the prefix workload: 1024 shared tokens, 128 sequences ---------------------

@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "e4m3"])
@pytest.mark.parametrize("append", [False, True], ids=["decode", "fused"])
def test_prefix_workload(fp8, append):
    w = W.prefix()
    sb = w.shared_tokens // w.block_size
    assert B.validate_shared_prefix(w.block_tables, w.context_lens, w.block_size, sb,
                                    append=True) == 0
    say(f"shared prefix workload: {sb} blocks, B={w.num_seqs}, fp8={fp8}, append={append}")
    got, kc, vc = run_shared(w, sb, fp8=fp8, append=append)
    rk, rv = oracle_caches(w, fp8)
    if append:
        assert np.array_equal(kc, rk) and np.array_equal(vc, rv), "caches differ from oracle"
    assert np.all(np.isfinite(f64(got, w.dtype)))
    check_close(got, oracle_rows(w, rk, rv, fp8), w.dtype, "prefix")


# ---- ragged shapes ------------------------------------------------------------------

SHAPES = [
    # (G, D, bs, dtype, batch, prefix tokens, private max)
    (4, 128, 16, W.BF16, 37, 512, 300),     # 32 tiles: exactly one chunk
    (1, 64, 8, W.F16, 70, 40, 90),          # 5 blocks of 8: 2 shared tiles, 1 block private
    (2, 128, 32, W.BF16, 9, 1600, 200),     # 100 tiles: 4 chunks, the last partial
    (8, 128, 8, W.F16, 5, 1032, 50),        # odd blocks (129) at bs 8
    (16, 64, 16, W.BF16, 3, 16, 700),       # one shared tile, one sequence per group
    (3, 128, 16, W.F16, 11, 256, 120),      # 5 sequences x 3 heads: padded columns
    (5, 64, 32, W.BF16, 1, 2048, 64),       # one sequence: half a column group
    (8, 64, 16, W.BF16, 64, 48, 17),        # three tiles, short private parts
]


@pytest.mark.parametrize("i", range(len(SHAPES)))
@pytest.mark.parametrize("pt", [0, 16, 64])
def test_shared_ragged_decode(i, pt):
    G, D, bs, dt, nseq, pre, pmax = SHAPES[i]
    g = np.random.default_rng(700 + i)
    hkv = int(g.integers(1, 3))
    lens = pre + g.integers(1, pmax + 1, size=nseq)
    w = W.build(f"sh{i}", lens, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                block_size=bs, dtype=dt, seed=800 + i, shared_prefix_tokens=pre,
                max_blocks_per_seq=(pre + pmax) // bs + 2)
    sb = pre // bs
    # some sequences attend over the prefix alone (no private token)
    cl = w.context_lens.copy()
    cl[::4] = pre
    assert B.validate_shared_prefix(w.block_tables, cl, bs, sb) == 0
    say(f"shared ragged {i}: G={G} D={D} bs={bs} {dt} Hkv={hkv} B={nseq} prefix={pre} pt={pt}")
    got, _, _ = run_shared(w, sb, cl=cl, pt=pt)
    rk, rv = oracle_caches(w, False)
    check_close(got, oracle_rows(w, rk, rv, False, cl), dt, f"shared ragged {i}")


@pytest.mark.parametrize("i", [0, 1, 3, 5])
def test_shared_ragged_fused(i):
    """The fused step over a shared prefix: the new tokens land in private
    blocks, both caches bit-exact, every row against the oracle."""
    G, D, bs, dt, nseq, pre, pmax = SHAPES[i]
    g = np.random.default_rng(900 + i)
    hkv = int(g.integers(1, 3))
    lens = pre + g.integers(1, pmax + 1, size=nseq)
    w = W.build(f"shf{i}", lens, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                block_size=bs, dtype=dt, seed=1000 + i, shared_prefix_tokens=pre,
                max_blocks_per_seq=(pre + pmax) // bs + 2)
    sb = pre // bs
    for fp8 in (False, True):
        say(f"shared fused {i}: G={G} D={D} bs={bs} B={nseq} fp8={fp8}")
        got, kc, vc = run_shared(w, sb, fp8=fp8, append=True, pt=16 if i % 2 else 0)
        rk, rv = oracle_caches(w, fp8)
        assert np.array_equal(kc, rk) and np.array_equal(vc, rv), "caches differ from oracle"
        check_close(got, oracle_rows(w, rk, rv, fp8), dt, f"shared fused {i} fp8={fp8}")


def test_zero_shared_blocks_is_plain_decode():
    w = W.llama8b()
    say("shared_blocks = 0 against paged_attention_decode")
    got, _, _ = run_shared(w, 0)
    kc, vc = caches(w, False, with_new=True)
    q = dev_bits(w.q, w.dtype)
    out = torch.empty_like(q)
    B.paged_attention_decode(out, q, kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                             torch.from_numpy(w.context_lens).to(DEV), w.scale, w.block_size,
                             w.num_kv_heads)
    torch.cuda.synchronize()
    assert np.array_equal(got, host_bits(out))


def test_shared_stages_equal_whole_call():
    """Split pass then merge as two calls equals one call, bit for bit."""
    w = W.prefix()
    sb = w.shared_tokens // w.block_size
    kc, vc = caches(w, False, with_new=True)
    q = dev_bits(w.q, w.dtype)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    outs = []
    for stages in ((3,), (1, 2)):
        out = torch.full_like(q, float("nan"))
        for st in stages:
            B.paged_attention_decode_shared(out, q, kc, vc, bt, cl, w.scale, w.block_size,
                                            w.num_kv_heads, sb, stages=st)
        torch.cuda.synchronize()
        outs.append(host_bits(out))
    assert np.array_equal(outs[0], outs[1])
