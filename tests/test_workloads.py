"""Host-side input generator and block manager (no GPU).

Pins the block manager against a hand-worked append/share example
(tests/golden/append_slots.json, derived from the BlockTable.append_token
description in "vLLM memory management and continuous batching from the
source", part 2, 2.1, and the shared-prefix description in "vLLM framework
analysis: how PagedAttention speeds up LLM inference 20x", 2.3), and checks
determinism, distributions and the bf16 rounding against torch's own cast.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from pagedattention_kv_cache_paged_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "append_slots.json")


def test_append_golden():
    g = json.load(open(GOLDEN))
    alloc = W.BlockAllocator(g["allocation_order"])
    t = W.BlockTable(alloc, g["block_size"])
    slots = [t.append_token() for _ in range(g["num_tokens"])]
    assert slots == g["expected_slots"]
    assert t.blocks == g["expected_blocks"]


def test_fork_golden():
    g = json.load(open(GOLDEN))
    alloc = W.BlockAllocator(g["allocation_order"])
    root = W.BlockTable(alloc, g["block_size"])
    for _ in range(g["fork_after"]):
        root.append_token()
    a, b = root.fork(), root.fork()
    assert {str(k): v for k, v in alloc.refcount.items()} == g["fork_expected_refcount"]
    assert [a.append_token(), b.append_token()] == g["fork_first_new_slot"]
    # releasing every holder returns the shared blocks to the pool
    for t in (root, a, b):
        t.free()
    assert alloc.refcount == {}
    assert sorted(alloc.free) == sorted(g["allocation_order"])


def test_fork_of_partial_block_refused():
    alloc = W.BlockAllocator(range(4))
    t = W.BlockTable(alloc, 4)
    for _ in range(5):
        t.append_token()
    with pytest.raises(ValueError):
        t.fork()


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(200000).astype(np.float32),
                        np.float32([0.0, -0.0, 1e-40, -1e-40, 3.0e38, 1.00390625, 1.01171875])])
    ours = W.to_bits(x, W.BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_f16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32)
    ours = W.to_bits(x, W.F16)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic():
    a, b = W.tiny(), W.tiny()
    for f in ("context_lens", "block_tables", "q", "token_k", "token_v", "token_slot"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_tiny_shape():
    w = W.tiny()
    assert w.context_lens.tolist() == [1, 17, 33, 100]
    assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size) == (4, 2, 64, 16)
    assert w.num_blocks == 64
    used = sum(math.ceil(L / 16) for L in [1, 17, 33, 100])
    assert used == 13
    assert w.spare_block is not None
    # slots are unique and every sequence's tokens sit in its own blocks
    assert len(set(w.token_slot.tolist())) == w.token_slot.size
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        idx = w.seq_tokens[s]
        assert idx.size == L
        for t in range(L):
            assert w.token_slot[idx[t]] == w.block_tables[s, t // 16] * 16 + t % 16
        assert np.all(w.block_tables[s, math.ceil(L / 16):] == w.spare_block)


def test_block_size_sweep_shares_token_data():
    ws = [W.short(bs) for bs in (8, 16, 32)]
    for w in ws[1:]:
        np.testing.assert_array_equal(w.context_lens, ws[0].context_lens)
        np.testing.assert_array_equal(w.q, ws[0].q)
        np.testing.assert_array_equal(w.token_k, ws[0].token_k)
        np.testing.assert_array_equal(w.token_v, ws[0].token_v)
    lens = ws[0].context_lens
    assert lens.min() >= 1 and lens.max() <= 512
    assert 40 < lens.mean() < 60


def test_llama8b_shape():
    w = W.llama8b()
    L = w.context_lens
    assert w.num_seqs == 64 and L.min() >= 128 and L.max() <= 2048
    need = int(sum(math.ceil(int(x) / 16) for x in L))
    assert w.num_blocks == math.ceil(1.2 * need)
    assert w.max_blocks_per_seq == 128
    assert w.bytes_per_token == 4096


def test_prefix_sharing_structure():
    w = W.prefix()
    assert w.shared_tokens == 1024
    shared = w.block_tables[:, :64]
    assert np.all(shared == shared[0])
    for b in shared[0]:
        assert w.refcount[int(b)] == 128
    # private blocks are distinct across sequences
    priv = []
    for s in range(w.num_seqs):
        nb = math.ceil(int(w.context_lens[s]) / 16)
        priv += w.block_tables[s, 64:nb].tolist()
    assert len(priv) == len(set(priv))
    assert not set(priv) & set(shared[0].tolist())
    # the new token lands in a private block
    new_blocks = w.token_slot[w.new_index] // 16
    assert not set(new_blocks.tolist()) & set(shared[0].tolist())
    assert w.unique_tokens == 1024 + int((w.context_lens - 1024).sum())


def test_placement_seed_changes_only_placement():
    a = W.build("a", [5, 40, 17], num_heads=4, num_kv_heads=2, head_dim=64, block_size=8,
                dtype=W.BF16, seed=7)
    b = W.build("b", [5, 40, 17], num_heads=4, num_kv_heads=2, head_dim=64, block_size=8,
                dtype=W.BF16, seed=7, placement_seed=99)
    np.testing.assert_array_equal(a.token_k, b.token_k)
    np.testing.assert_array_equal(a.q, b.q)
    assert not np.array_equal(a.block_tables, b.block_tables)
