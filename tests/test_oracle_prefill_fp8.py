"""Pins of the oracle's chunked prefill over E4M3 caches (no GPU).

The FP8 reading of "vLLM framework analysis: how PagedAttention speeds up LLM
inference 20x" (intelliparadigm.com), 7 (an E4M3 KV cache, one scale per
tensor, code * scale), applied to the chunked prefill of "vLLM core
architecture overview" (5688vip.com), 4.3.  Pinned against:

* torch's scaled_dot_product_attention in fp64 on each sequence's logical K
  and V, dequantised by torch's own float8_e4m3fn decoder times the scales
  and gathered through the harness's block tables (explicit chunk masks);
* the 16-bit prefill oracle, bit for bit, on E4M3-exact token values with
  scales that are powers of two (the 16-bit caches hold code * scale);
* oracle_decode_fp8: a one-row chunk equals it bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import workloads as W

F8 = torch.float8_e4m3fn


def f64(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(F8).to(
        torch.float64).numpy()


def fp8_setup(lengths, chunks, hq, hkv, d, bs, dtype, seed, ks, vs):
    w = W.build("pf8", lengths, num_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                dtype=dtype, seed=seed)
    kc, vc = w.nan_caches_fp8()
    oracle.kv_write_fp8(w.token_k, w.token_v, w.token_slot, kc, vc, bs, dtype, ks, vs)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    g = np.random.default_rng(seed + 1)
    q = W.normal_bits(g, (int(qs[-1]), hq, d), dtype)
    return w, kc, vc, q, qs


def sdpa_fp8(w, kc, vc, q, qs, chunks, ks, vs):
    """Reference from the dequantised caches, read through the block tables."""
    bs, G = w.block_size, w.num_heads // w.num_kv_heads
    kval = e4m3_values(kc.reshape(-1)).reshape(kc.shape) * ks
    vval = e4m3_values(vc.reshape(-1)).reshape(vc.shape) * vs
    out = np.zeros(q.shape, np.float64)
    for s in range(w.num_seqs):
        n = chunks[s]
        if n == 0:
            continue
        L = int(w.context_lens[s])
        blocks = [w.block_tables[s][t // bs] for t in range(L)]
        K = np.stack([kval[blocks[t], :, t % bs, :] for t in range(L)], 1)   # [Hkv, L, D]
        V = np.stack([vval[blocks[t], :, (t % bs) // 4, :, t % 4] for t in range(L)], 1)
        k = torch.from_numpy(K).repeat_interleave(G, 0)
        v = torch.from_numpy(V).repeat_interleave(G, 0)
        qq = torch.from_numpy(f64(q[qs[s]:qs[s] + n], w.dtype)).permute(1, 0, 2)
        pos = np.arange(L - n, L)
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        o = torch.nn.functional.scaled_dot_product_attention(qq, k, v, attn_mask=mask,
                                                             scale=w.scale)
        out[qs[s]:qs[s] + n] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("bs,dtype", [(8, W.BF16), (16, W.F16), (32, W.BF16)])
def test_fp8_prefill_equals_dequantised_sdpa(bs, dtype):
    ks, vs = 0.03, 0.05
    lengths, chunks = [1, 40, 97, 70], [1, 40, 13, 0]
    w, kc, vc, q, qs = fp8_setup(lengths, chunks, 8, 2, 64, bs, dtype, 70 + bs, ks, vs)
    got = oracle.prefill_fp8(q, kc, vc, w.block_tables, w.context_lens, qs, w.scale, bs,
                             dtype, ks, vs)
    ref = sdpa_fp8(w, kc, vc, q, qs, chunks, ks, vs)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.25, 2.0)])
def test_fp8_prefill_equals_16bit_oracle_on_e4m3_exact_data(ks, vs):
    """Token values that are E4M3 values: with power-of-two scales the 16-bit
    caches can hold code * scale exactly, so both oracles see the same
    numbers."""
    lengths, chunks = [30, 100, 7], [30, 17, 7]
    w = W.build("pf8x", lengths, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                dtype=W.BF16, seed=44)
    g = np.random.default_rng(6)
    vals = e4m3_values(np.arange(0x60))
    pick = lambda shape: (vals[g.integers(0, 0x60, size=shape)] *
                          g.choice([-1.0, 1.0], size=shape))
    kv = pick(w.token_k.shape)
    vv = pick(w.token_v.shape)
    k8, v8 = w.nan_caches_fp8()
    w.token_k = W.to_bits(kv.astype(np.float32), W.BF16)
    w.token_v = W.to_bits(vv.astype(np.float32), W.BF16)
    oracle.kv_write_fp8(w.token_k, w.token_v, w.token_slot, k8, v8, 16, W.BF16, 1.0, 1.0)
    k16, v16 = w.nan_caches()
    kb = W.to_bits((kv * ks).astype(np.float32), W.BF16)
    vb = W.to_bits((vv * vs).astype(np.float32), W.BF16)
    oracle.kv_write(kb, vb, w.token_slot, k16, v16, 16)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = W.normal_bits(np.random.default_rng(7), (int(qs[-1]), 4, 64), W.BF16)
    a = oracle.prefill(q, k16, v16, w.block_tables, w.context_lens, qs, w.scale, 16, W.BF16)
    b = oracle.prefill_fp8(q, k8, v8, w.block_tables, w.context_lens, qs, w.scale, 16, W.BF16,
                           ks, vs)
    assert np.array_equal(a, b)


def test_fp8_one_row_chunk_equals_decode():
    ks, vs = 0.04, 0.02
    w, kc, vc, q, qs = fp8_setup([50, 9], [1, 1], 8, 4, 64, 16, W.F16, 90, ks, vs)
    got = oracle.prefill_fp8(q, kc, vc, w.block_tables, w.context_lens, qs, w.scale, 16,
                             W.F16, ks, vs)
    ref = oracle.decode_fp8(q, kc, vc, w.block_tables, w.context_lens, w.scale, 16, W.F16,
                            ks, vs)
    assert np.array_equal(got, ref)
