"""GPU parity of paged_attention_prefill (chunked prefill) through the C ABI
against oracle_prefill: |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| element by
element, on ragged batches mixing whole prompts, chunks after a cached
prefix (prefix and chunk lengths off tile and block edges), one-row chunks
and empty chunks, over head_dim, block size, GQA group (1 to 16) and dtype;
and a Llama-3-8B-shaped chunk batch (sampled rows); bfloat16 V beyond
binary16's range, which takes the kernel's exact mode.  Rows outside the
chunks are never written.  paged_attention_prefill_fp8 is held to the same
bar against oracle_prefill_fp8 on E4M3 caches that paged_kv_write_fp8
filled (the reading of "vLLM framework analysis: how PagedAttention speeds
up LLM inference 20x", 7)."""
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


def say(msg):
    print(msg, flush=True)


def f64(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dev_bits(bits, dtype):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(TD[dtype])


def run(lengths, chunks, G, hkv, d, bs, dtype, seed, rows=None, v_scale=None, kv8=None,
        v_map=None, **wkw):
    """kv8 = (k_scale, v_scale): E4M3 caches and paged_attention_prefill_fp8.
    v_map: a function of the tokens' V values [N, Hkv, D] (float64) giving
    the V values to store (rounded to the cache type)."""
    w = W.build("pf", lengths, num_heads=G * hkv, num_kv_heads=hkv, head_dim=d,
                block_size=bs, dtype=dtype, seed=seed, **wkw)
    if v_scale is not None:  # V values times v_scale, kept inside +-65000
        v = np.clip(f64(w.token_v, dtype) * v_scale, -65000.0, 65000.0)
        w.token_v = W.to_bits(v.astype(np.float32), dtype).reshape(w.token_v.shape)
    if v_map is not None:
        v = v_map(f64(w.token_v, dtype))
        w.token_v = W.to_bits(v.astype(np.float32), dtype).reshape(w.token_v.shape)
    ksh, vsh = w.cache_shapes()
    if kv8 is None:
        nan = int(np.array([W.NAN_BITS[dtype]], np.uint16).view(np.int16)[0])
        kc = torch.full(ksh, nan, dtype=torch.int16, device=DEV).view(TD[dtype])
        vc = torch.full(vsh, nan, dtype=torch.int16, device=DEV).view(TD[dtype])
        okc, ovc = w.nan_caches()
    else:
        kc = torch.full(ksh, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        vc = torch.full(vsh, W.FP8_NAN, dtype=torch.uint8, device=DEV)
        okc, ovc = w.nan_caches_fp8()
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        kd, vd, sd = dev_bits(k, dtype), dev_bits(v, dtype), torch.from_numpy(s).to(DEV)
        if kv8 is None:
            B.paged_kv_write(kd, vd, sd, kc, vc)
            oracle.kv_write(k, v, s, okc, ovc, bs)
        else:
            B.paged_kv_write_fp8(kd, vd, sd, kc, vc, *kv8)
            oracle.kv_write_fp8(k, v, s, okc, ovc, bs, dtype, *kv8)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    g = np.random.default_rng(seed + 7)
    q = W.normal_bits(g, (int(qs[-1]), w.num_heads, d), dtype)
    qd = dev_bits(q, dtype)
    out = torch.full_like(qd, float("nan"))
    say(f"prefill{'_fp8' if kv8 else ''} B={len(lengths)} G={G} hkv={hkv} D={d} bs={bs} "
        f"{dtype} rows={qs[-1]}")
    meta = (torch.from_numpy(w.block_tables).to(DEV), torch.from_numpy(w.context_lens).to(DEV),
            torch.from_numpy(qs).to(DEV), w.scale)
    mq = max(chunks) if len(chunks) else 0
    if kv8 is None:
        B.paged_attention_prefill(out, qd, kc, vc, *meta, bs, hkv, mq)
    else:
        B.paged_attention_prefill_fp8(out, qd, kc, vc, *meta, *kv8, bs, hkv, mq)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)

    def ref_of(qr, bt, cl, qsr):
        if kv8 is None:
            return oracle.prefill(qr, okc, ovc, bt, cl, qsr, w.scale, bs, dtype)
        return oracle.prefill_fp8(qr, okc, ovc, bt, cl, qsr, w.scale, bs, dtype, *kv8)

    if rows is None:
        return got, ref_of(q, w.block_tables, w.context_lens, qs), None
    # sampled rows: the oracle over those rows only (each row on its own)
    ref = np.zeros((len(rows), w.num_heads, d))
    seq_of = np.searchsorted(qs, rows, side="right") - 1
    for j, (r, s) in enumerate(zip(rows, seq_of)):
        L = int(w.context_lens[s])
        p = L - (qs[s + 1] - qs[s]) + (r - qs[s])
        ref[j] = ref_of(q[r:r + 1], w.block_tables[s:s + 1], np.array([p + 1], np.int32),
                        np.array([0, 1], np.int32))[0]
    return got[rows], ref, None


def check(got, ref, dtype, what, atol=ATOL):
    g = f64(got, dtype)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = ~(err <= atol + RTOL * np.abs(ref))
    say(f"  {what} max_abs={err.max():.3e} n={ref.size}")
    assert not bad.any(), f"{what}: {bad.sum()} out of tolerance, worst {err[bad].max():.3e}"


CASES = []
for i, (G, d, bs, dt) in enumerate([(1, 64, 16, W.F16), (2, 128, 8, W.BF16), (3, 64, 32, W.BF16),
                                    (4, 128, 16, W.BF16), (5, 64, 8, W.F16), (8, 128, 32, W.F16),
                                    (16, 64, 16, W.BF16), (4, 64, 32, W.F16), (1, 128, 8, W.BF16)]):
    CASES.append((i, G, d, bs, dt))


@pytest.mark.parametrize("i,G,d,bs,dt", CASES)
def test_prefill_ragged(i, G, d, bs, dt):
    g = np.random.default_rng(900 + i)
    lengths = [1, 17, 64, 130, 200, 97, 33, 300]
    chunks = [1, 17, 64, 66, 1, 0, 20, 129]   # whole prompts, prefix + chunk, one row, none
    hkv = int(g.integers(1, 3))
    got, ref, _ = run(lengths, chunks, G, hkv, d, bs, dt, 1000 + i)
    check(got, ref, dt, f"ragged{i}")


def test_prefill_long_prompt_and_edges():
    """A whole 1000-token prompt (many key tiles, 16 query blocks), a chunk
    that starts mid-tile, and chunk lengths one either side of 64."""
    got, ref, _ = run([1000, 511, 95, 65], [1000, 200, 63, 65], 4, 2, 128, 16, W.BF16, 77)
    check(got, ref, W.BF16, "long")


def test_prefill_llama8b_chunks():
    """Llama-3-8B shape: 4 sequences, 512-token chunks after 1536 cached
    tokens (32 q / 8 kv heads, head_dim 128, bf16, block 16); sampled rows."""
    g = np.random.default_rng(5)
    rows = np.sort(g.choice(4 * 512, 48, replace=False))
    got, ref, _ = run([2048] * 4, [512] * 4, 4, 8, 128, 16, W.BF16, 55, rows=rows)
    check(got, ref, W.BF16, "llama8b chunks")


@pytest.mark.parametrize("d,dt", [(64, W.F16), (128, W.BF16)])
def test_prefill_table_at_limit(d, dt):
    """A 32768-token context at block size 8 fills the 4096 block ids a
    workgroup keeps on chip (with D = 128 the workgroup's LDS is then 84 KB);
    a 70-row chunk at its end (sampled rows) and a short whole prompt beside
    it."""
    g = np.random.default_rng(8)
    rows = np.sort(np.concatenate([g.choice(70, 10, replace=False), [70, 71, 75]]))
    got, ref, _ = run([32768, 6], [70, 6], 2, 1, d, 8, dt, 31, rows=rows,
                      max_blocks_per_seq=4096)
    check(got, ref, dt, f"table at limit D={d}")


@pytest.mark.parametrize("log2s", [14, -20])
def test_prefill_bf16_v_range(log2s):
    """bfloat16 V runs through binary16 in P.V: V scaled by 2^14 (values up to
    about 65000, converted exactly) keeps the tolerance in units of V's
    scale; V scaled by 2^-20 (binary16 subnormals, rounded by < 2^-24) keeps
    the absolute one."""
    s = 2.0 ** log2s
    got, ref, _ = run([300, 77, 129], [300, 40, 1], 4, 2, 128, 16, W.BF16, 91 + log2s,
                      v_scale=s)
    check(got, ref, W.BF16, f"v x 2^{log2s}", atol=ATOL * max(s, 1.0))


@pytest.mark.parametrize("log2s", [17, 60, 125])
def test_prefill_bf16_v_beyond_binary16(log2s):
    """bfloat16 V beyond binary16's range (unit-normal V times 2^17, 2^60,
    2^125; 2^125 reaches within a factor 2 of bfloat16's largest value):
    every workgroup stages such values and recomputes its rows in the exact
    mode (bfloat16 V, weights as bfloat16 hi + lo), so the tolerance holds in
    units of V's scale, where saturation at 65504 would miss by orders of
    magnitude."""
    s = 2.0 ** log2s
    got, ref, _ = run([300, 77, 129], [300, 40, 1], 4, 2, 128, 16, W.BF16, 191 + log2s,
                      v_map=lambda v: v * s)
    check(got, ref, W.BF16, f"v x 2^{log2s}", atol=ATOL * s)


@pytest.mark.parametrize("G,d", [(4, 128), (1, 64), (2, 128)])
def test_prefill_bf16_v_mixed_magnitudes(G, d):
    """Among unit-normal V, six tokens carry V of 2^100 times a unit normal's
    magnitude.  Workgroups that stage one of them take the exact mode, also
    for their rows that attend only to unit-scale V (those before the huge
    token, or in another head), which must keep the absolute tolerance of
    unit V; rows that see a huge token are dominated by it (relative
    tolerance).  Workgroups that stage none keep the binary16 path."""
    g = np.random.default_rng(40 + G)

    def v_map(v):
        idx = g.choice(v.shape[0], 6, replace=False)
        v = v.copy()
        v[idx] = np.abs(v[idx]) * 2.0 ** 100
        return v

    got, ref, _ = run([300, 150, 129, 64], [300, 100, 1, 64], G, 2, d, 16, W.BF16, 300 + G,
                      v_map=v_map)
    check(got, ref, W.BF16, f"mixed G={G} d={d}")


def test_prefill_leaves_other_rows():
    """Rows past every chunk (the tail of q / out) are not written, and a
    chunk longer than its context gets no rows."""
    w = W.build("pfx", [40, 30], num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                dtype=W.F16, seed=3)
    ksh, vsh = w.cache_shapes()
    kc = torch.zeros(ksh, dtype=torch.float16, device=DEV)
    vc = torch.zeros(vsh, dtype=torch.float16, device=DEV)
    for which in ("hist", "new"):
        k, v, s = w.write_batch(which)
        B.paged_kv_write(dev_bits(k, W.F16), dev_bits(v, W.F16), torch.from_numpy(s).to(DEV),
                         kc, vc)
    q = torch.randn(80, 4, 64, dtype=torch.float16, device=DEV)
    out = torch.full_like(q, 7.0)
    qs = torch.tensor([0, 10, 45], dtype=torch.int32, device=DEV)   # seq 1: 35 rows > 30 tokens
    B.paged_attention_prefill(out, q, kc, vc, torch.from_numpy(w.block_tables).to(DEV),
                              torch.from_numpy(w.context_lens).to(DEV), qs, w.scale, 16, 2, 35)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.all(o[10:] == 7.0)
    assert np.all(np.isfinite(o[:10])) and not np.all(o[:10] == 7.0)


KS8, VS8 = 0.02, 0.03   # N(0, 1) data: codes stay well inside +-448


@pytest.mark.parametrize("i,G,d,bs,dt", CASES[:6])
def test_prefill_fp8_ragged(i, G, d, bs, dt):
    g = np.random.default_rng(950 + i)
    lengths = [1, 17, 64, 130, 200, 97, 33, 300]
    chunks = [1, 17, 64, 66, 1, 0, 20, 129]
    hkv = int(g.integers(1, 3))
    got, ref, _ = run(lengths, chunks, G, hkv, d, bs, dt, 2000 + i, kv8=(KS8, VS8))
    check(got, ref, dt, f"fp8 ragged{i}")


def test_prefill_fp8_llama8b_chunks():
    """The Llama-3-8B chunk batch over E4M3 caches; sampled rows."""
    g = np.random.default_rng(6)
    rows = np.sort(g.choice(4 * 512, 48, replace=False))
    got, ref, _ = run([2048] * 4, [512] * 4, 4, 8, 128, 16, W.BF16, 56, rows=rows,
                      kv8=(KS8, VS8))
    check(got, ref, W.BF16, "fp8 llama8b chunks")


@pytest.mark.parametrize("ks,vs", [(1.0 / 64, 2.0 ** -6), (0.5, 7.0)])
def test_prefill_fp8_scales(ks, vs):
    """Other scales: with 2^-6 the codes reach a few hundred (near E4M3's
    448); with 0.5 and 7 they are small, and with 7 about a tenth of the V
    codes are subnormal (below 2^-6).  The dequantized values keep the data's size, and so does
    out: the tolerance is unchanged."""
    got, ref, _ = run([150, 77], [150, 9], 2, 2, 64, 16, W.F16, 70, kv8=(ks, vs))
    check(got, ref, W.F16, f"fp8 ks={ks} vs={vs}")
