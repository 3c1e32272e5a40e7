"""Seeded synthetic workloads for paged decode attention.

This module draws inputs and plays the host-side block manager; it holds none
of the attention arithmetic, so both the HIP path and the fp64 oracle may use
it.  What it does:

* draws context lengths, physical block placement and token data from three
  independent, seeded ``numpy.random.Generator`` streams (lengths, placement,
  data), so that two workloads that differ only in placement or block size
  carry bit-identical token data;
* rounds N(0, 1) float32 draws to binary16 / bfloat16 bit patterns with
  round-to-nearest-even;
* allocates physical blocks the way the append step of "vLLM memory
  management and continuous batching from the source"
  (developer.cloud.tencent.cn), part 2, 2.1, describes: a sequence takes a
  new block from the pool exactly when the number of tokens it already stores
  is a multiple of the block size, and each token's slot is that block's
  number times the block size plus the offset inside it;
* shares prefix blocks between sequences by reference with reference counts,
  as "vLLM framework analysis: how PagedAttention speeds up LLM inference 20x"
  (intelliparadigm.com), 2.3, describes for a common system prompt;
* pads block-table entries past a sequence's last block with the number of a
  block that no sequence uses, which consumers fill with NaN.

The five named workloads follow the configurations this library is measured
on (tiny fp16 case; Llama-3-8B-shaped decode; short-request sweep over block
sizes; shared system prompt; 32k-token long context).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

F16 = "f16"
BF16 = "bf16"
NAN_BITS = {F16: 0x7E00, BF16: 0x7FC0}
FP8_NAN = 0x7F  # E4M3 (e4m3fn) NaN code
ELEM_BYTES = 2

_STREAM_LENGTHS, _STREAM_PLACEMENT, _STREAM_DATA = 0, 1, 2


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round finite float32 values to binary16 / bfloat16 bits (nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype != BF16:
        raise ValueError(dtype)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    chunk = 1 << 24
    for i in range(0, flat_in.size, chunk):
        u = flat_in[i:i + chunk].view(np.uint32)
        if not np.all((u & 0x7F800000) != 0x7F800000):
            raise ValueError("to_bits expects finite values")
        flat_out[i:i + chunk] = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
                                 >> np.uint32(16)).astype(np.uint16)
    return out


def normal_bits(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) float32 draws rounded to ``dtype`` bits, drawn in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    chunk = 1 << 24
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        out[i:i + m] = to_bits(g.standard_normal(m, dtype=np.float32), dtype)
    return out.reshape(shape)


# ---- host-side block manager ----------------------------------------------

class BlockAllocator:
    """Free list over a fixed pool of physical blocks, with reference counts."""

    def __init__(self, order: Sequence[int]):
        self.free: List[int] = [int(b) for b in order][::-1]  # pop() takes order[0] first
        self.refcount = {}

    def allocate(self) -> int:
        if not self.free:
            raise MemoryError("block pool exhausted")
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> int:
        self.refcount[b] += 1
        return b

    def release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            del self.refcount[b]
            self.free.append(b)


class BlockTable:
    """Logical-to-physical block map of one sequence plus its fill count."""

    def __init__(self, allocator: BlockAllocator, block_size: int):
        self.alloc = allocator
        self.block_size = block_size
        self.blocks: List[int] = []
        self.num_tokens = 0

    def append_token(self) -> int:
        """Reserve the next token position; returns its slot."""
        bs = self.block_size
        if self.num_tokens % bs == 0:
            self.blocks.append(self.alloc.allocate())
        slot = self.blocks[self.num_tokens // bs] * bs + self.num_tokens % bs
        self.num_tokens += 1
        return slot

    def fork(self) -> "BlockTable":
        """A new sequence that shares every block of this one by reference.
        Only whole blocks may be shared (the fork never writes into them)."""
        if self.num_tokens % self.block_size:
            raise ValueError("sharing a partly filled block needs copy-on-write")
        child = BlockTable(self.alloc, self.block_size)
        child.blocks = [self.alloc.share(b) for b in self.blocks]
        child.num_tokens = self.num_tokens
        return child

    def free(self) -> None:
        for b in self.blocks:
            self.alloc.release(b)
        self.blocks = []
        self.num_tokens = 0


# ---- workload -------------------------------------------------------------

@dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    num_blocks: int
    max_blocks_per_seq: int
    context_lens: np.ndarray          # int32 [B]
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq]
    q: np.ndarray                     # uint16 [B, Hq, D]
    token_k: np.ndarray               # uint16 [N, Hkv, D], every stored token once
    token_v: np.ndarray               # uint16 [N, Hkv, D]
    token_slot: np.ndarray            # int64 [N]
    seq_tokens: List[np.ndarray]      # per sequence: indices into token_* in logical order
    shared_tokens: int = 0
    refcount: dict = field(default_factory=dict)
    spare_block: Optional[int] = None

    # -- derived views (pure bookkeeping) --
    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def new_index(self) -> np.ndarray:
        """Token index of each sequence's newest token (the one appended by
        this decode step)."""
        return np.array([t[-1] for t in self.seq_tokens], dtype=np.int64)

    @property
    def hist_index(self) -> np.ndarray:
        new = set(self.new_index.tolist())
        return np.array([i for i in range(self.token_slot.size) if i not in new],
                        dtype=np.int64)

    def write_batch(self, which: str):
        """(k, v, slot_mapping) for the history tokens ("hist") or this step's
        new tokens ("new")."""
        idx = self.hist_index if which == "hist" else self.new_index
        return (np.ascontiguousarray(self.token_k[idx]),
                np.ascontiguousarray(self.token_v[idx]),
                np.ascontiguousarray(self.token_slot[idx]))

    def seq_kv(self, s: int):
        """Logical K and V of sequence s, [L, Hkv, D] bits, position order."""
        idx = self.seq_tokens[s]
        return self.token_k[idx], self.token_v[idx]

    @property
    def logical_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    @property
    def unique_tokens(self) -> int:
        return int(self.token_slot.size)

    @property
    def bytes_per_token(self) -> int:
        """K plus V bytes of one context token over all KV heads."""
        return 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES

    def cache_shapes(self):
        nb, h, bs, d = self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim
        return (nb, h, bs, d), (nb, h, bs // 4, d, 4)

    def nan_caches(self):
        """Host K and V caches filled with the dtype's NaN."""
        ks, vs = self.cache_shapes()
        nan = np.uint16(NAN_BITS[self.dtype])
        return np.full(ks, nan, dtype=np.uint16), np.full(vs, nan, dtype=np.uint16)

    def nan_caches_fp8(self):
        """Host E4M3 K and V caches (one byte per element) filled with NaN."""
        ks, vs = self.cache_shapes()
        return (np.full(ks, FP8_NAN, dtype=np.uint8), np.full(vs, FP8_NAN, dtype=np.uint8))


def build(name: str, lengths: Sequence[int], *, num_heads: int, num_kv_heads: int,
          head_dim: int, block_size: int, dtype: str, seed: int,
          pool="1.2x", max_blocks_per_seq: Optional[int] = None,
          shared_prefix_tokens: int = 0, placement_seed: Optional[int] = None,
          placement: str = "random", scale: Optional[float] = None) -> Workload:
    """Generic builder.  ``lengths`` are the context lengths after this step's
    token is appended (so each is at least 1).  With ``shared_prefix_tokens``
    = P > 0, every sequence's first P tokens are one shared set of blocks.
    ``placement="identity"`` hands blocks out in increasing order, so each
    sequence's blocks are physically consecutive (a contiguous cache)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    B = lengths.size
    bs = block_size
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if shared_prefix_tokens:
        if shared_prefix_tokens % bs:
            raise ValueError("shared prefix must be whole blocks")
        if np.any(lengths <= shared_prefix_tokens):
            raise ValueError("each sequence needs a private token after the prefix")
    if np.any(lengths < 0):
        raise ValueError("negative length")
    need = int(sum(math.ceil((int(L) - shared_prefix_tokens) / bs) for L in lengths))
    need += shared_prefix_tokens // bs
    if pool == "1.2x":
        num_blocks = int(math.ceil(1.2 * need))
    elif pool == "need":
        num_blocks = need
    else:
        num_blocks = int(pool)
    if num_blocks < need:
        raise ValueError("pool too small")
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(math.ceil(int(lengths.max(initial=0)) / bs)))
    if np.any(np.ceil(lengths / bs) > max_blocks_per_seq):
        raise ValueError("block table too narrow")

    seed_p = seed if placement_seed is None else placement_seed
    if placement == "identity":
        order = np.arange(num_blocks)
    elif placement == "random":
        order = rng(seed_p, _STREAM_PLACEMENT).permutation(num_blocks)
    else:
        raise ValueError(placement)
    alloc = BlockAllocator(order)

    # token stream: shared prefix once, then each sequence's private tokens
    slots: List[int] = []
    seq_tokens: List[np.ndarray] = []
    tables: List[BlockTable] = []
    prefix_idx: List[int] = []
    if shared_prefix_tokens:
        root = BlockTable(alloc, bs)
        for _ in range(shared_prefix_tokens):
            prefix_idx.append(len(slots))
            slots.append(root.append_token())
    for s in range(B):
        if shared_prefix_tokens:
            t = root.fork()
            idx = list(prefix_idx)
        else:
            t = BlockTable(alloc, bs)
            idx = []
        while t.num_tokens < lengths[s]:
            idx.append(len(slots))
            slots.append(t.append_token())
        tables.append(t)
        seq_tokens.append(np.array(idx, dtype=np.int64))
    if shared_prefix_tokens:
        root.free()  # the prompt's own table goes; sequences keep the blocks

    spare = alloc.free[-1] if alloc.free else None
    bt = np.empty((B, max_blocks_per_seq), dtype=np.int32)
    for s, t in enumerate(tables):
        pad = spare if spare is not None else (t.blocks[-1] if t.blocks else 0)
        bt[s, :] = pad
        bt[s, :len(t.blocks)] = t.blocks

    g = rng(seed, _STREAM_DATA)
    n_tok = len(slots)
    q = normal_bits(g, (B, num_heads, head_dim), dtype)
    token_k = normal_bits(g, (n_tok, num_kv_heads, head_dim), dtype)
    token_v = normal_bits(g, (n_tok, num_kv_heads, head_dim), dtype)

    return Workload(
        name=name, dtype=dtype, num_seqs=B, num_heads=num_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs,
        scale=float(1.0 / math.sqrt(head_dim)) if scale is None else float(scale),
        num_blocks=num_blocks, max_blocks_per_seq=max_blocks_per_seq,
        context_lens=lengths.astype(np.int32), block_tables=bt, q=q,
        token_k=token_k, token_v=token_v,
        token_slot=np.array(slots, dtype=np.int64), seq_tokens=seq_tokens,
        shared_tokens=shared_prefix_tokens, refcount=dict(alloc.refcount),
        spare_block=spare)


# ---- the five named workloads ---------------------------------------------

def tiny(seed: int = 1) -> Workload:
    """Batch 4, context lengths {1, 17, 33, 100}, 4 query / 2 KV heads,
    head_dim 64, block 16, pool of 64 blocks, fp16."""
    return build("tiny", [1, 17, 33, 100], num_heads=4, num_kv_heads=2, head_dim=64,
                 block_size=16, dtype=F16, seed=seed, pool=64, max_blocks_per_seq=7)


def llama8b(seed: int = 2, block_size: int = 16, placement: str = "random") -> Workload:
    """Llama-3-8B-shaped single-layer decode: batch 64, 32 query / 8 KV heads,
    head_dim 128, bf16, block 16, lengths uniform in [128, 2048], pool 1.2x.
    ``placement="identity"`` gives each sequence physically consecutive
    blocks (a contiguous cache) with the same token data."""
    lengths = rng(seed, _STREAM_LENGTHS).integers(128, 2048, size=64, endpoint=True)
    return build("llama8b", lengths, num_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=block_size, dtype=BF16, seed=seed,
                 max_blocks_per_seq=2048 // block_size, placement=placement)


def short(block_size: int = 16, seed: int = 3) -> Workload:
    """Batch 256 short requests, lengths geometric with mean 50 clipped to
    [1, 512], 8B head shape, fp16; token data independent of block size."""
    lengths = rng(seed, _STREAM_LENGTHS).geometric(1.0 / 50.0, size=256)
    lengths = np.clip(lengths, 1, 512)
    return build(f"short_bs{block_size}", lengths, num_heads=32, num_kv_heads=8,
                 head_dim=128, block_size=block_size, dtype=F16, seed=seed,
                 max_blocks_per_seq=512 // block_size)


def prefix(seed: int = 4) -> Workload:
    """Batch 128 sharing one 1024-token system prompt (64 blocks of 16) by
    reference, then 32..512 private tokens each; bf16, 8B head shape."""
    suffix = rng(seed, _STREAM_LENGTHS).integers(32, 512, size=128, endpoint=True)
    return build("prefix", 1024 + suffix, num_heads=32, num_kv_heads=8, head_dim=128,
                 block_size=16, dtype=BF16, seed=seed, shared_prefix_tokens=1024,
                 max_blocks_per_seq=(1024 + 512) // 16)


def long(seed: int = 5) -> Workload:
    """Batch 8 at 32768 tokens each, 64 query / 8 KV heads (70B layer),
    head_dim 128, bf16, block 16, pool exactly the need, random placement."""
    return build("long", [32768] * 8, num_heads=64, num_kv_heads=8, head_dim=128,
                 block_size=16, dtype=BF16, seed=seed, pool="need",
                 max_blocks_per_seq=2048)


NAMED = {"tiny": tiny, "llama8b": llama8b, "short": short, "prefix": prefix, "long": long}
