"""GPU parity of the FP8 (E4M3) cache path through the C ABI.

The reading ("vLLM framework analysis: how PagedAttention speeds up LLM
inference 20x", 7: FP8 for attention, FP16 elsewhere) and the oracle are
described in tests/test_oracle_fp8.py.  Here:

* paged_kv_write_fp8: bit-exact against the oracle over both whole caches
  (NaN sentinels in untouched slots survive), on random tokens at several
  scales, on crafted values (exact rounding ties, saturation, subnormal
  codes, zeros of both signs) and with padding slots;
* paged_attention_decode_fp8: |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| on the
  named workloads (every output row, the oracle's rows shared out over host
  threads), ragged shapes over head_dim, block size, GQA group and q type,
  and the split edge cases (empty sequences, more waves than tiles).
"""
import math

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
KS, VS = 0.02, 0.03  # N(0, 1) data: codes stay well inside +-448


def say(msg):
    print(msg, flush=True)


def dev_bits(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(TD[dtype])


def f64(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_close(got_bits, ref, dtype, what=""):
    g = f64(got_bits, dtype)
    err = np.abs(g - ref)
    bad = ~(err <= ATOL + RTOL * np.abs(ref))
    say(f"  {what} max_abs={err.max():.3e} n={ref.size}")
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, worst {err[bad].max():.3e}"


class Case8:
    """Device E4M3 caches of one workload, filled through paged_kv_write_fp8."""

    def __init__(self, w, ks=KS, vs=VS, with_new=True):
        self.w, self.ks, self.vs = w, ks, vs
        ksh, vsh = w.cache_shapes()
        self.kc = torch.full(ksh, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        self.vc = torch.full(vsh, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        for which in (("hist", "new") if with_new else ("hist",)):
            k, v, s = w.write_batch(which)
            if s.size:
                B.paged_kv_write_fp8(dev_bits(k, w.dtype), dev_bits(v, w.dtype),
                                     torch.from_numpy(s).to(DEV), self.kc, self.vc, ks, vs)
        self.q = dev_bits(w.q, w.dtype)
        self.bt = torch.from_numpy(w.block_tables).to(DEV)
        self.cl = torch.from_numpy(w.context_lens).to(DEV)

    def decode(self, partition_tokens=0, cl=None):
        w = self.w
        out = torch.empty_like(self.q)
        B.paged_attention_decode_fp8(out, self.q, self.kc, self.vc, self.bt,
                                     self.cl if cl is None else cl, w.scale, self.ks, self.vs,
                                     w.block_size, w.num_kv_heads,
                                     partition_tokens=partition_tokens)
        torch.cuda.synchronize()
        return out.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_caches8(w, ks=KS, vs=VS):
    kc, vc = w.nan_caches_fp8()
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        oracle.kv_write_fp8(k, v, s, kc, vc, w.block_size, w.dtype, ks, vs)
    return kc, vc


NAMED = [("tiny", W.tiny), ("short_bs8", lambda: W.short(8)), ("short_bs32", lambda: W.short(32)),
         ("llama8b", W.llama8b), ("prefix", W.prefix), ("long", W.long)]


@pytest.mark.parametrize("name,make", NAMED, ids=[n for n, _ in NAMED])
def test_write_fp8_bit_exact(name, make):
    say(f"fp8 write {name}")
    w = make()
    c = Case8(w)
    torch.cuda.synchronize()
    kc, vc = oracle_caches8(w)
    assert np.array_equal(c.kc.cpu().numpy(), kc)
    assert np.array_equal(c.vc.cpu().numpy(), vc)


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.0371, 0.5), (3.0, 0.001)])
def test_write_fp8_crafted_values(dtype, ks, vs):
    """Exact rounding ties of the E4M3 grid, the saturation range, subnormal
    codes and signed zeros, through the kernel's own encoder."""
    codes = np.arange(0x7F)
    vals = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    extra = np.array([448.0, 449.0, 464.0, 500.0, 1e4, 2.0 ** -10, 3 * 2.0 ** -11, 0.0, -0.0,
                      2.0 ** -9, 0.015625], np.float32)
    x = np.concatenate([vals, mids, extra, -vals, -mids, -extra]).astype(np.float32) * ks
    D = 64
    n = -(-x.size // (2 * D)) * 2 * D
    x = np.concatenate([x, np.zeros(n - x.size, np.float32)])
    T = n // (2 * D)                       # tokens of 2 kv heads x 64 dims
    bits = W.to_bits(x, dtype).reshape(T, 2, D)
    vbits = W.to_bits((x / ks * vs).astype(np.float32), dtype).reshape(T, 2, D)
    bs, nb = 16, 8
    slots = np.random.default_rng(9).permutation(nb * bs)[:T].astype(np.int64)
    slots[3] = -1                          # padding
    kc = torch.full((nb, 2, bs, D), W.FP8_NAN, dtype=torch.uint8, device=DEV)
    vc = torch.full((nb, 2, bs // 4, D, 4), W.FP8_NAN, dtype=torch.uint8, device=DEV)
    B.paged_kv_write_fp8(dev_bits(bits, dtype), dev_bits(vbits, dtype),
                         torch.from_numpy(slots).to(DEV), kc, vc, ks, vs)
    torch.cuda.synchronize()
    okc = np.full((nb, 2, bs, D), W.FP8_NAN, np.uint8)
    ovc = np.full((nb, 2, bs // 4, D, 4), W.FP8_NAN, np.uint8)
    oracle.kv_write_fp8(bits, vbits, slots, okc, ovc, bs, dtype, ks, vs)
    assert np.array_equal(kc.cpu().numpy(), okc)
    assert np.array_equal(vc.cpu().numpy(), ovc)


@pytest.mark.parametrize("name,make", [
    ("tiny", W.tiny), ("short_bs8", lambda: W.short(8)), ("short_bs16", lambda: W.short(16)),
    ("short_bs32", lambda: W.short(32)), ("llama8b", W.llama8b), ("prefix", W.prefix),
    ("long", W.long),
], ids=["tiny", "short_bs8", "short_bs16", "short_bs32", "llama8b", "prefix", "long"])
def test_decode_fp8_named(name, make):
    """Every output row of each named workload over E4M3 caches."""
    w = make()
    say(f"fp8 decode {name}")
    got = Case8(w).decode()
    kc, vc = oracle_caches8(w)
    assert np.all(np.isfinite(f64(got, w.dtype)))
    rows = oracle.all_rows(w.num_seqs, w.num_heads)
    ref = oracle.decode_fp8_rows(rows, w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                 w.block_size, w.dtype, KS, VS, threads=oracle.host_threads())
    check_close(got, ref.reshape(got.shape), w.dtype, name)


SHAPES = [(1, 64, 8, W.F16), (2, 128, 16, W.BF16), (4, 64, 32, W.BF16), (8, 128, 8, W.F16),
          (16, 128, 16, W.BF16), (3, 128, 32, W.F16), (5, 64, 16, W.BF16)]


@pytest.mark.parametrize("i", range(len(SHAPES)))
@pytest.mark.parametrize("pt", [0, 32])
def test_decode_fp8_ragged(i, pt):
    G, D, bs, dt = SHAPES[i]
    g = np.random.default_rng(3000 + i)
    hkv = int(g.integers(1, 4))
    lens = np.concatenate([[1, 2, 15, 16, 17, 31, 33], g.integers(1, 700, size=5)])
    w = W.build(f"f8rag{i}", lens, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                block_size=bs, dtype=dt, seed=4000 + i,
                max_blocks_per_seq=int(math.ceil(700 / bs)) + 2)
    say(f"fp8 ragged {i}: G={G} D={D} bs={bs} {dt} Hkv={hkv} pt={pt}")
    ks, vs = 0.0123 * (i + 1), 0.5 / (i + 1)
    got = Case8(w, ks, vs).decode(partition_tokens=pt)
    kc, vc = oracle_caches8(w, ks, vs)
    ref = oracle.decode_fp8(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, bs, dt,
                            ks, vs)
    check_close(got, ref, dt, f"fp8 ragged{i}")


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_decode_fp8_split_edges(bs):
    lens = [0, 1, 0, 16, 17, 0, 300, 31, 32, 33, 0, 5, 64, 0]
    w = W.build("f8edges", [max(L, 1) for L in lens], num_heads=8, num_kv_heads=2,
                head_dim=64, block_size=bs, dtype=W.BF16, seed=95 + bs,
                max_blocks_per_seq=(320 + bs - 1) // bs)
    c = Case8(w)
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    kc, vc = oracle_caches8(w)
    ref = oracle.decode_fp8(w.q, kc, vc, w.block_tables, np.array(lens, np.int32), w.scale,
                            bs, w.dtype, KS, VS)
    for pt in (0, 16, 1024):
        say(f"fp8 edges bs={bs} pt={pt}")
        got = c.decode(partition_tokens=pt, cl=cl)
        assert np.all(f64(got, w.dtype)[np.array(lens) == 0] == 0)
        check_close(got, ref, w.dtype, f"fp8 edges bs{bs} pt{pt}")
