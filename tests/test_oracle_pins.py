"""Pins of the fp64 oracle against things other than itself (no GPU).

The pages print no attention values, so the oracle's decode is pinned by
closed forms, a library routine it must reduce to, brute force, and
invariants the paging idea fixes:

* element decoders: every binary16 / bfloat16 bit pattern against numpy's
  float16 and torch's bfloat16 conversions;
* append: round trip through the block tables built by the host block
  manager, untouched slots stay NaN, repeated / out-of-range slots refused;
* identity (contiguous) placement and random placement equal dense
  attention from torch's scaled_dot_product_attention in fp64 (with GQA by
  repeat_interleave), i.e. paging only changes where K and V live
  ("vLLM memory management and continuous batching from the source",
  part 2, 2.3);
* brute force in numpy from the logical arrays on random tiny shapes;
* physical placement permutation, block size and shared-vs-private prefix
  blocks leave the result bit-identical ("vLLM core architecture overview",
  4.1; "vLLM framework analysis ... 20x", 2.3);
* closed forms: context length 1 returns that token's V, identical keys (or
  q = 0, or scale = 0) return the mean of V, a hand-worked three-token case,
  a dominant logit returns its V, logits near 1000 do not overflow;
* the split-context log-sum-exp merge equals the single pass.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from pagedattention_kv_cache_paged_amd import workloads as W


# ---- helpers ----------------------------------------------------------------

def fill(w, with_new=True):
    kc, vc = w.nan_caches()
    k, v, s = w.write_batch("hist")
    oracle.kv_write(k, v, s, kc, vc, w.block_size)
    if with_new:
        k, v, s = w.write_batch("new")
        oracle.kv_write(k, v, s, kc, vc, w.block_size)
    return kc, vc


def run(w, kc=None, vc=None, tables=None):
    if kc is None:
        kc, vc = fill(w)
    bt = w.block_tables if tables is None else tables
    return oracle.decode(w.q, kc, vc, bt, w.context_lens, w.scale, w.block_size, w.dtype)


def lib_decode(bits, dtype):
    """Decode bits with numpy's own float16 / a float32 reinterpretation
    (bfloat16 is the upper half of a binary32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == W.F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dense_numpy(w):
    """Brute force from the logical arrays, no cache, no block table."""
    G = w.group
    out = np.zeros((w.num_seqs, w.num_heads, w.head_dim))
    for s in range(w.num_seqs):
        K, V = (lib_decode(a, w.dtype) for a in w.seq_kv(s))
        for h in range(w.num_heads):
            q = lib_decode(w.q[s, h], w.dtype)
            x = (K[:, h // G, :] @ q) * w.scale
            p = np.exp(x - x.max())
            out[s, h] = (p[:, None] * V[:, h // G, :]).sum(0) / p.sum()
    return out


def dense_sdpa(w):
    """torch scaled_dot_product_attention in float64 on the CPU."""
    G = w.group
    out = np.zeros((w.num_seqs, w.num_heads, w.head_dim))
    for s in range(w.num_seqs):
        K, V = (torch.from_numpy(lib_decode(a, w.dtype)) for a in w.seq_kv(s))
        K = K.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        V = V.permute(1, 0, 2).repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        q = torch.from_numpy(lib_decode(w.q[s], w.dtype)).unsqueeze(0).unsqueeze(2)
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=w.scale)
        out[s] = o[0, :, 0, :].numpy()
    return out


def rel_err(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---- element decoders ---------------------------------------------------------

def test_f16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([oracle.f16_to_f64(b) for b in bits])
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decoder_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([oracle.bf16_to_f64(b) for b in bits])
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


# ---- append -------------------------------------------------------------------

@pytest.mark.parametrize("bs", [8, 16, 32])
def test_write_round_trip(bs):
    w = W.build("rt", [1, 9, 40, 33], num_heads=6, num_kv_heads=3, head_dim=64,
                block_size=bs, dtype=W.BF16, seed=11)
    kc, vc = fill(w)
    nan = W.NAN_BITS[w.dtype]
    touched_k = np.zeros(kc.shape, bool)
    touched_v = np.zeros(vc.shape, bool)
    for s in range(w.num_seqs):
        K, V = w.seq_kv(s)
        for t in range(int(w.context_lens[s])):
            b, o = w.block_tables[s, t // bs], t % bs
            np.testing.assert_array_equal(kc[b, :, o, :], K[t])
            np.testing.assert_array_equal(vc[b, :, o // 4, :, o % 4], V[t])
            touched_k[b, :, o, :] = True
            touched_v[b, :, o // 4, :, o % 4] = True
    assert np.all(kc[~touched_k] == nan) and np.all(vc[~touched_v] == nan)


def test_write_skips_negative_slots():
    w = W.tiny()
    kc, vc = w.nan_caches()
    k, v, s = w.write_batch("new")
    s = s.copy()
    s[1] = -1
    oracle.kv_write(k, v, s, kc, vc, w.block_size)
    nan = W.NAN_BITS[w.dtype]
    for i in range(4):
        b, o = divmod(int(w.write_batch("new")[2][i]), w.block_size)
        assert np.all(kc[b, :, o, :] == nan) == (i == 1)


@pytest.mark.parametrize("bad", ["dup", "range"])
def test_write_rejects_bad_slots(bad):
    w = W.tiny()
    kc, vc = w.nan_caches()
    k, v, s = w.write_batch("new")
    s = s.copy()
    if bad == "dup":
        s[2] = s[0]
    else:
        s[3] = w.num_blocks * w.block_size
    with pytest.raises(oracle.OracleError):
        oracle.kv_write(k, v, s, kc, vc, w.block_size)
    assert np.all(kc == W.NAN_BITS[w.dtype]) and np.all(vc == W.NAN_BITS[w.dtype])


# ---- decode against dense attention -------------------------------------------

@pytest.mark.parametrize("placement", ["identity", "random"])
@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_decode_equals_sdpa(placement, dtype):
    w = W.build("sdpa", [1, 16, 17, 64, 100], num_heads=8, num_kv_heads=2, head_dim=64,
                block_size=16, dtype=dtype, seed=21, placement=placement,
                max_blocks_per_seq=8)
    if placement == "identity":
        # blocks of each sequence are consecutive: a contiguous cache
        for s in range(w.num_seqs):
            n = math.ceil(int(w.context_lens[s]) / 16)
            row = w.block_tables[s, :n]
            assert np.all(np.diff(row) == 1)
    assert rel_err(run(w), dense_sdpa(w)) <= 1e-12


def test_decode_llama_group_equals_sdpa():
    w = W.build("sdpa8", [130, 257], num_heads=32, num_kv_heads=8, head_dim=128,
                block_size=16, dtype=W.BF16, seed=22)
    assert rel_err(run(w), dense_sdpa(w)) <= 1e-12


@pytest.mark.parametrize("trial", range(12))
def test_decode_brute_force_tiny(trial):
    g = np.random.default_rng(100 + trial)
    B = int(g.integers(1, 4))
    lens = g.integers(1, 41, size=B)
    bs = int(g.choice([8, 16, 32]))
    hkv = int(g.choice([1, 2]))
    G = int(g.choice([1, 2, 4, 8, 16]))
    D = int(g.choice([64, 128]))
    dtype = W.F16 if trial % 2 else W.BF16
    w = W.build("bf", lens, num_heads=hkv * G, num_kv_heads=hkv, head_dim=D,
                block_size=bs, dtype=dtype, seed=200 + trial)
    out = run(w)
    assert np.all(np.isfinite(out))  # NaN-filled slots and padding never reached
    assert rel_err(out, dense_numpy(w)) <= 1e-12


def test_tiny_workload_brute_force():
    w = W.tiny()
    assert rel_err(run(w), dense_numpy(w)) <= 1e-12


# ---- invariants of paging --------------------------------------------------------

def test_placement_permutation_bit_identical():
    a = W.build("p", [3, 50, 129, 77], num_heads=8, num_kv_heads=4, head_dim=64,
                block_size=16, dtype=W.BF16, seed=31)
    outs = [run(a)]
    for ps in (1, 2, 3):
        b = W.build("p", [3, 50, 129, 77], num_heads=8, num_kv_heads=4, head_dim=64,
                    block_size=16, dtype=W.BF16, seed=31, placement_seed=1000 + ps)
        assert not np.array_equal(a.block_tables, b.block_tables)
        outs.append(run(b))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_block_size_bit_identical():
    lens = [1, 8, 9, 31, 32, 33, 200]
    outs = [run(W.build("b", lens, num_heads=4, num_kv_heads=2, head_dim=128, block_size=bs,
                        dtype=W.F16, seed=41)) for bs in (8, 16, 32)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_shared_prefix_equals_private_copies():
    bs, P = 16, 64
    w = W.build("pre", [P + 5, P + 40, P + 17], num_heads=8, num_kv_heads=2, head_dim=64,
                block_size=bs, dtype=W.BF16, seed=51, shared_prefix_tokens=P)
    shared = w.block_tables[:, :P // bs]
    assert np.all(shared == shared[0])
    out_shared = run(w)
    # same logical data, each sequence given private blocks of its own
    need = sum(math.ceil(int(L) / bs) for L in w.context_lens)
    nb = need + 1
    alloc = W.BlockAllocator(np.random.default_rng(5).permutation(nb))
    kc, vc = (np.full(s, W.NAN_BITS[w.dtype], np.uint16) for s in
              ((nb, 2, bs, 64), (nb, 2, bs // 4, 64, 4)))
    tables = np.full((w.num_seqs, w.max_blocks_per_seq), alloc.free[0], np.int32)
    for s in range(w.num_seqs):
        t = W.BlockTable(alloc, bs)
        slots = np.array([t.append_token() for _ in range(int(w.context_lens[s]))])
        K, V = w.seq_kv(s)
        oracle.kv_write(K, V, slots, kc, vc, bs)
        tables[s, :len(t.blocks)] = t.blocks
    out_private = oracle.decode(w.q, kc, vc, tables, w.context_lens, w.scale, bs, w.dtype)
    assert np.array_equal(out_shared, out_private)


def test_nan_poison_not_reached():
    w = W.tiny()
    kc, vc = fill(w)
    # also point every padded table entry at the (NaN-filled) spare block
    assert np.all(kc[w.spare_block] == W.NAN_BITS[w.dtype])
    assert np.all(np.isfinite(run(w, kc, vc)))


# ---- closed forms -----------------------------------------------------------------

def _single(dtype, K_rows, V_rows, q_row, scale, bs=16):
    """A one-sequence, one-head case laid out by the block manager."""
    L, D = len(K_rows), len(q_row)
    w = W.build("cf", [L], num_heads=1, num_kv_heads=1, head_dim=D, block_size=bs,
                dtype=dtype, seed=61, scale=scale)
    w.q[0, 0] = W.to_bits(np.float32(q_row), dtype)
    w.token_k[:, 0, :] = W.to_bits(np.float32(K_rows), dtype)
    w.token_v[:, 0, :] = W.to_bits(np.float32(V_rows), dtype)
    return w, run(w)[0, 0]


def test_length_one_returns_v():
    w = W.tiny()  # sequence 0 has a single token
    out = run(w)
    _, V = w.seq_kv(0)
    for h in range(w.num_heads):
        assert np.array_equal(out[0, h], lib_decode(V[0, h // w.group], w.dtype))


@pytest.mark.parametrize("mode", ["same_keys", "zero_q", "zero_scale"])
def test_uniform_weights_give_mean_v(mode):
    g = np.random.default_rng(71)
    L, D = 37, 64
    K = g.standard_normal((L, D)).astype(np.float32)
    if mode == "same_keys":
        K[:] = K[0]
    V = g.standard_normal((L, D)).astype(np.float32)
    q = np.zeros(D, np.float32) if mode == "zero_q" else g.standard_normal(D).astype(np.float32)
    scale = 0.0 if mode == "zero_scale" else 0.125
    w, out = _single(W.BF16, K, V, q, scale)
    Vd = lib_decode(W.to_bits(V, W.BF16), W.BF16)
    np.testing.assert_allclose(out, Vd.mean(0), rtol=0, atol=1e-14)


def test_hand_worked_three_tokens():
    # logits 0, 1, 2 (scale 1): weights 1, e, e^2
    K = [[0, 0], [1, 0], [2, 0]]
    V = [[1, 0], [0, 1], [1, 1]]
    _, out = _single(W.F16, K, V, [1, 0], 1.0)
    e = math.e
    z = 1 + e + e * e
    np.testing.assert_allclose(out, [(1 + e * e) / z, (e + e * e) / z], rtol=1e-15)


def test_dominant_logit_and_no_overflow():
    D = 64
    g = np.random.default_rng(81)
    K = g.standard_normal((20, D)).astype(np.float32) * 0.01
    K[13, 0] = 60.0  # logit ~60 above the rest with q = e_0, scale 1
    V = g.standard_normal((20, D)).astype(np.float32)
    q = np.zeros(D, np.float32)
    q[0] = 1.0
    _, out = _single(W.BF16, K, V, q, 1.0)
    Vd = lib_decode(W.to_bits(V, W.BF16), W.BF16)
    np.testing.assert_allclose(out, Vd[13], rtol=0, atol=1e-20 + 20 * math.exp(-59))
    # adding 1024 to every logit changes nothing (the maximum is taken out
    # before exponentiating; exp(1084) would overflow a double)
    q2 = q * 16.0
    q2[1] = 16.0
    K2 = K.copy()
    K2[:, 1] = 1024.0  # scale * 16 * 1024 = +1024 on every logit
    _, out2 = _single(W.BF16, K2, V, q2, 1.0 / 16.0)
    assert np.all(np.isfinite(out2))
    np.testing.assert_allclose(out2, Vd[13], rtol=0, atol=1e-20 + 20 * math.exp(-59))


def test_zero_length_gives_zeros():
    w = W.tiny()
    kc, vc = fill(w)
    cl = w.context_lens.copy()
    cl[2] = 0
    out = oracle.decode(w.q, kc, vc, w.block_tables, cl, w.scale, w.block_size, w.dtype)
    assert np.all(out[2] == 0) and np.all(np.isfinite(out))


# ---- split-context merge ------------------------------------------------------------

@pytest.mark.parametrize("part", [8, 16, 48, 256, 4096])
def test_partitioned_merge_equals_single_pass(part):
    w = W.build("part", [1, 100, 333], num_heads=4, num_kv_heads=2, head_dim=64,
                block_size=8, dtype=W.BF16, seed=91)
    kc, vc = fill(w)
    full = run(w, kc, vc)
    for s in range(w.num_seqs):
        for h in range(w.num_heads):
            o = oracle.decode_row_partitioned(s, h, part, w.q, kc, vc, w.block_tables,
                                              w.context_lens, w.scale, w.block_size, w.dtype)
            assert rel_err(o, full[s, h]) <= 1e-12


def test_rows_equal_full():
    w = W.tiny()
    kc, vc = fill(w)
    full = run(w, kc, vc)
    rows = [(3, 1), (0, 0), (2, 3)]
    got = oracle.decode_rows(rows, w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                             w.block_size, w.dtype)
    for i, (s, h) in enumerate(rows):
        assert np.array_equal(got[i], full[s, h])


@pytest.mark.parametrize("threads", [2, 3, 8])
def test_pooled_rows_equal_full(threads):
    """Rows shared out over host threads (how the GPU tests check every row
    of the large workloads) equal the single full call, bit for bit."""
    w = W.build("pool", [1, 17, 33, 100, 250, 5, 64], num_heads=8, num_kv_heads=2,
                head_dim=64, block_size=16, dtype=W.BF16, seed=17)
    kc, vc = fill(w)
    full = run(w, kc, vc)
    rows = oracle.all_rows(w.num_seqs, w.num_heads)
    assert rows.shape == (w.num_seqs * w.num_heads, 2)
    assert np.array_equal(rows[w.num_heads + 3], [1, 3])
    got = oracle.decode_rows(rows, w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                             w.block_size, w.dtype, threads=threads)
    assert np.array_equal(got.reshape(full.shape), full)


# ---- metadata errors --------------------------------------------------------------------

def test_bad_block_id_refused():
    w = W.tiny()
    kc, vc = fill(w)
    bt = w.block_tables.copy()
    bt[3, 2] = w.num_blocks
    with pytest.raises(oracle.OracleError):
        oracle.decode(w.q, kc, vc, bt, w.context_lens, w.scale, w.block_size, w.dtype)


def test_length_beyond_table_refused():
    w = W.tiny()
    kc, vc = fill(w)
    cl = w.context_lens.copy()
    cl[0] = w.max_blocks_per_seq * w.block_size + 1
    with pytest.raises(oracle.OracleError):
        oracle.decode(w.q, kc, vc, w.block_tables, cl, w.scale, w.block_size, w.dtype)
