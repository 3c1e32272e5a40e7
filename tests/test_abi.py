"""C-ABI library on the CPU: it loads, exports every function
include/paged_attn.h declares, and rejects bad arguments on the host
before anything is launched (no call here reaches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch  # noqa: F401  (the binding binds to torch's HIP runtime)

from pagedattention_kv_cache_paged_amd import binding as B
from pagedattention_kv_cache_paged_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")

FAKE = 0x100000  # aligned non-null address; never dereferenced in these tests


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    names = declared_functions()
    assert {"paged_kv_write", "paged_attention_decode", "paged_attention_decode_ex",
            "paged_attention_decode_stages", "paged_attention_workspace_bytes",
            "paged_attention_split_waves", "paged_validate_metadata", "pa_strerror",
            "pa_abi_version", "paged_kv_write_fp8", "paged_attention_decode_fp8",
            "paged_attention_decode_append", "paged_attention_decode_append_stages",
            "paged_attention_decode_append_noalloc", "paged_attention_decode_shared",
            "paged_attention_workspace_bytes_shared", "paged_validate_shared_prefix",
            "paged_attention_prefill",
            "paged_validate_prefill", "paged_attention_prefill_fp8"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pa_abi_version() == 9


def test_single_hip_runtime():
    B.load()
    assert len(B.hip_runtimes_mapped()) == 1


def test_strerror():
    lib = B.load()
    for code in range(-8, 1):
        assert lib.pa_strerror(code) and lib.pa_strerror(code) != b"unknown error"
    assert lib.pa_strerror(-99) == b"unknown error"


def _decode(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.125, bs=16, hkv=8,
             B=4, hq=32, d=128, mb=128, nb=1000, dtype=1, pt=0, ws=FAKE, wsb=1 << 30,
             stages=3, stream=None)
    a.update(kw)
    return B.load().paged_attention_decode_stages(
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"], a["bs"], a["hkv"],
        a["B"], a["hq"], a["d"], a["mb"], a["nb"], a["dtype"], a["pt"], a["ws"], a["wsb"],
        a["stages"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -2),
    (dict(d=96), -3),
    (dict(bs=4), -3),
    (dict(bs=64), -3),
    (dict(hq=30), -3),               # not a multiple of the KV heads
    (dict(hq=8 * 32), -3),           # group of 32 > 16
    (dict(B=-1), -3),
    (dict(B=70000), -3),
    (dict(B=8193), -3),              # tile prefix of more sequences than LDS holds
    (dict(B=8192, mb=300000), -3),   # 2.46e9 tiles per KV head: past the int32 tile prefix
    (dict(B=4, mb=600000000), -3),   # a table wider than int32 positions
    (dict(mb=0), -3),
    (dict(nb=0), -3),
    (dict(scale=float("nan")), -3),
    (dict(pt=24), -3),               # not a multiple of 16
    (dict(pt=40, bs=8), -3),
    (dict(pt=16 * 64 + 16), -3),     # more tiles per wave than lanes
    (dict(stages=0), -3),
    (dict(stages=4), -3),
    (dict(out=None), -1),
    (dict(bt=None), -1),
    (dict(q=FAKE + 8), -7),
    (dict(out=FAKE + 2), -7),
    (dict(ws=None), -4),
    (dict(wsb=1024), -4),
    (dict(ws=FAKE + 4), -7),
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code


def test_decode_zero_seqs_is_noop():
    assert _decode(B=0, out=None, q=None) == 0


def _write(**kw):
    a = dict(k=FAKE, v=FAKE, slots=FAKE, kc=FAKE, vc=FAKE, T=4, hkv=8, d=128, bs=16, nb=100,
             dtype=0, stream=None)
    a.update(kw)
    return B.load().paged_kv_write(a["k"], a["v"], a["slots"], a["kc"], a["vc"], a["T"],
                                   a["hkv"], a["d"], a["bs"], a["nb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), -2),
    (dict(d=80), -3),
    (dict(bs=12), -3),
    (dict(T=-1), -3),
    (dict(T=1 << 31), -3),
    (dict(hkv=0), -3),
    (dict(nb=0), -3),
    (dict(k=None), -1),
    (dict(vc=None), -1),
    (dict(v=FAKE + 2), -7),
    (dict(slots=FAKE + 4), -7),
])
def test_write_rejects(kw, code):
    assert _write(**kw) == code


def test_write_zero_tokens_is_noop():
    assert _write(T=0, k=None) == 0


@pytest.mark.parametrize("ks,vs,code", [(0.0, 1.0, -3), (1.0, -2.0, -3), (float("inf"), 1.0, -3),
                                       (1.0, float("nan"), -3), (1e-39, 1.0, -3),
                                       (0.5, 0.25, 0)])
def test_fp8_scales_checked(ks, vs, code):
    lib = B.load()
    rc = lib.paged_kv_write_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 0 if code == 0 else 4, 8, 128, 16,
                                100, 1, ks, vs, None)
    assert rc == code
    rc = lib.paged_attention_decode_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0.125, ks, vs, 16, 8,
                                        0 if code == 0 else 4, 32, 128, 128, 1000, 1, 0, FAKE,
                                        1 << 30, 3, None)
    assert rc == code


def test_split_and_workspace():
    """Hand-worked split sizes: cap = seqs * ceil(max_blocks * bs / 16) tiles
    per KV head; waves = max(ceil(1024 / Hkv) or ceil(cap * 16 / pt),
    ceil(cap / 64)), at most cap."""
    assert B.split_waves(4, 2, 7, 16) == 28          # cap 28 < 512
    assert B.split_waves(64, 8, 128, 16) == 128      # cap 8192: 1024 / 8
    assert B.split_waves(8, 8, 2048, 16) == 256      # cap 16384: 64 tiles per wave
    assert B.split_waves(256, 8, 64, 8) == 128       # cap 256 * 32
    assert B.split_waves(64, 8, 128, 16, 256) == 512  # 8192 * 16 / 256
    assert B.split_waves(64, 8, 128, 16, 1024) == 128
    assert B.split_waves(3, 1, 64, 32, 16) == 384    # cap 3 * 128, one tile each
    assert B.split_waves(64, 8, 128, 16, 24) == 0    # not a multiple of 16
    assert B.split_waves(64, 8, 128, 16, 2048) == 0  # over 64 tiles
    # llama8b sizes: 128 waves + 64 seqs = 192 slots per query head;
    # partials 32 x 192 x 128 fp32, (m, l) 32 x 192 x 2 fp32, prefix 65 int32
    # padded to 512 B
    assert B.workspace_bytes(64, 32, 8, 128, 128, 16) == (
        32 * 192 * 128 * 4 + 32 * 192 * 2 * 4 + 512)
    assert B.workspace_bytes(64, 32, 8, 128, 128, 16, 2048) == 0
    assert B.workspace_bytes(0, 32, 8, 128, 128, 16) == 0
    # the batch limit: 8192 sequences (lengths and tile prefix in LDS)
    assert B.workspace_bytes(8192, 4, 2, 64, 3, 16) > 0
    assert B.workspace_bytes(8193, 4, 2, 64, 3, 16) == 0
    # the split pass's tile prefix is int32: at most 2^31 - 1 tiles per KV head
    # (8192 sequences x 262143 tiles fits; x 262145 does not)
    assert B.split_waves(8192, 8, 262143, 16) > 0
    assert B.workspace_bytes(8192, 32, 8, 128, 262143, 16) > 0
    assert B.split_waves(8192, 8, 262145, 16) == 0
    assert B.workspace_bytes(8192, 32, 8, 128, 262145, 16) == 0


def test_validate_metadata():
    w = W.tiny()
    k, v, s = w.write_batch("hist")
    assert B.validate_metadata(w.block_tables, w.context_lens, 16, w.num_blocks, s) == 0
    bt = w.block_tables.copy()
    bt[3, 0] = w.num_blocks
    assert B.validate_metadata(bt, w.context_lens, 16, w.num_blocks) == -6
    # entries past the used blocks are not checked
    bt = w.block_tables.copy()
    bt[0, 5] = -7
    assert B.validate_metadata(bt, w.context_lens, 16, w.num_blocks) == 0
    cl = w.context_lens.copy()
    cl[1] = 7 * 16 + 1
    assert B.validate_metadata(w.block_tables, cl, 16, w.num_blocks) == -6
    s2 = s.copy()
    s2[5] = s2[4]
    assert B.validate_metadata(w.block_tables, w.context_lens, 16, w.num_blocks, s2) == -6
    s2 = s.copy()
    s2[5] = w.num_blocks * 16
    assert B.validate_metadata(w.block_tables, w.context_lens, 16, w.num_blocks, s2) == -6
    s2 = s.copy()
    s2[5] = -1
    assert B.validate_metadata(w.block_tables, w.context_lens, 16, w.num_blocks, s2) == 0


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(2, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        B.paged_attention_decode(q.clone(), q, torch.zeros(4, 2, 16, 64, dtype=torch.float16),
                                 torch.zeros(4, 2, 64, 16, dtype=torch.float16),
                                 torch.zeros(2, 1, dtype=torch.int32),
                                 torch.ones(2, dtype=torch.int32), 0.125, 16, 2)


def _append(**kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.125,
             ks=1.0, vs=1.0, bs=16, hkv=8, B=4, hq=32, d=128, mb=128, nb=1000, dtype=1, fp8=0,
             pt=0, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(kw)
    return B.load().paged_attention_decode_append(
        a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"],
        a["ks"], a["vs"], a["bs"], a["hkv"], a["B"], a["hq"], a["d"], a["mb"], a["nb"],
        a["dtype"], a["fp8"], a["pt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), -1), (dict(vn=None), -1), (dict(out=None), -1),
    (dict(kn=FAKE + 2), -7), (dict(vn=FAKE + 1), -7),
    (dict(fp8=2), -2), (dict(dtype=3), -2),
    (dict(fp8=1, ks=0.0), -3), (dict(fp8=1, vs=float("nan")), -3),
    (dict(d=96), -3), (dict(bs=12), -3), (dict(hq=30), -3),
    (dict(wsb=16), -4), (dict(ws=None), -4),
])
def test_append_rejects_before_launch(kw, code):
    assert _append(**kw) == code


def test_append_zero_sequences_is_noop():
    assert _append(B=0, out=None, q=None, kn=None, vn=None) == 0


def _shared(**kw):
    a = dict(out=FAKE, q=FAKE, kn=None, vn=None, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE,
             scale=0.125, ks=1.0, vs=1.0, bs=16, hkv=8, B=4, hq=32, d=128, mb=128, nb=1000,
             dtype=1, fp8=0, sb=64, pt=0, ws=FAKE, wsb=1 << 30, stages=3, stream=None)
    a.update(kw)
    return B.load().paged_attention_decode_shared(
        a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"],
        a["ks"], a["vs"], a["bs"], a["hkv"], a["B"], a["hq"], a["d"], a["mb"], a["nb"],
        a["dtype"], a["fp8"], a["sb"], a["pt"], a["ws"], a["wsb"], a["stages"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(sb=-1), -3), (dict(sb=129), -3),          # outside the table
    (dict(kn=FAKE), -1), (dict(vn=FAKE), -1),       # one of the new rows only
    (dict(fp8=2), -2), (dict(stages=4), -3), (dict(d=96), -3),
    (dict(wsb=16), -4), (dict(ws=None), -4),
])
def test_shared_rejects_before_launch(kw, code):
    assert _shared(**kw) == code


def test_shared_workspace_sizes():
    """Hand-worked: the prefix workload (128 sequences, 32 q / 8 kv heads,
    D 128, 96-entry tables, 64 shared blocks of 16).  Private tiles at most
    128 x 32 = 4096 per KV head: 128 waves (1024 / 8), 256 slots per query
    head; the 64 shared tiles are 2 chunks of 32, partials 32 x 128 x 2."""
    slots = 128 + 128
    private = 32 * slots * 128 * 4 + 32 * slots * 2 * 4 + 768  # prefix of 129 int32 -> 768 B
    shared = 32 * 128 * 2 * 128 * 4 + 32 * 128 * 2 * 2 * 4
    assert B.workspace_bytes_shared(128, 32, 8, 128, 96, 16, 64) == private + shared
    # no shared blocks: the plain decode's workspace
    assert B.workspace_bytes_shared(64, 32, 8, 128, 128, 16, 0) == \
        B.workspace_bytes(64, 32, 8, 128, 128, 16)
    assert B.workspace_bytes_shared(128, 32, 8, 128, 96, 16, 97) == 0


def test_validate_shared_prefix():
    w = W.prefix()
    bt, cl = w.block_tables.copy(), w.context_lens.copy()
    assert B.validate_shared_prefix(bt, cl, 16, 64) == 0
    assert B.validate_shared_prefix(bt, cl, 16, 64, append=True) == 0
    assert B.validate_shared_prefix(bt, cl, 16, 0) == 0
    assert B.validate_shared_prefix(bt, cl, 16, 65) == -6   # block 64 is private
    bt2 = bt.copy()
    bt2[7, 13] = bt2[7, 70]
    assert B.validate_shared_prefix(bt2, cl, 16, 64) == -6
    cl2 = cl.copy()
    cl2[3] = 1024
    assert B.validate_shared_prefix(bt, cl2, 16, 64) == 0   # the prefix alone
    assert B.validate_shared_prefix(bt, cl2, 16, 64, append=True) == -6
    cl2[3] = 1023
    assert B.validate_shared_prefix(bt, cl2, 16, 64) == -6
    assert B.validate_shared_prefix(bt, cl, 16, -1) == -3


def _noalloc(**kw):
    a = dict(out=FAKE, q=FAKE, kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, scale=0.125,
             ks=1.0, vs=1.0, bs=16, hkv=8, B=4, hq=32, d=128, mb=128, nb=1000, dtype=1, fp8=0,
             pt=0, stream=None)
    a.update(kw)
    return B.load().paged_attention_decode_append_noalloc(
        a["out"], a["q"], a["kn"], a["vn"], a["kc"], a["vc"], a["bt"], a["cl"], a["scale"],
        a["ks"], a["vs"], a["bs"], a["hkv"], a["B"], a["hq"], a["d"], a["mb"], a["nb"],
        a["dtype"], a["fp8"], a["pt"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    # 512 x 32 heads: 1536 partial slots of 128 fp32 per head, 25 MB > 16 MiB
    (dict(B=512), -8),
    # 128-token split of 8 full 32k-token sequences, 64 heads: 2056 slots, 67 MB
    (dict(B=8, hq=64, mb=2048, pt=128), -8),
    (dict(d=96), -3), (dict(bs=12), -3), (dict(pt=24), -3), (dict(dtype=3), -2),
])
def test_noalloc_rejects_before_launch(kw, code):
    """Sizes past the fixed scratch array are refused with PA_ERR_SCRATCH
    before the library touches the GPU; other bad sizes as for the step with
    a workspace."""
    assert _noalloc(**kw) == code


def test_noalloc_zero_sequences_is_noop():
    assert _noalloc(B=0, out=None, q=None, kn=None, vn=None) == 0


def test_noalloc_scratch_covers_named_workloads():
    """The fixed 16 MiB holds the workspace of every named workload."""
    for w in (W.tiny(), W.short(8), W.short(16), W.short(32)):
        assert 0 < B.workspace_bytes(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim,
                                     w.max_blocks_per_seq, w.block_size) <= B.SCRATCH_BYTES
    for args in ((64, 32, 8, 128, 128, 16),     # llama8b
                 (128, 32, 8, 128, 96, 16),     # prefix
                 (8, 64, 8, 128, 2048, 16)):    # long
        assert 0 < B.workspace_bytes(*args) <= B.SCRATCH_BYTES


def test_append_binding_checks_shapes():
    """The Python mirror rejects mismatched tensors before calling the
    library (CPU tensors never reach it: the device check comes first)."""
    q = torch.zeros(2, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        B.paged_attention_decode_append(q, q, q, q, q, q, q, q, 0.1, 16, 2)


def _prefill(**kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, qs=FAKE, scale=0.125, bs=16,
             hkv=8, B=4, hq=32, d=128, mb=128, nb=1000, dtype=1, mq=512, stream=None)
    a.update(kw)
    return B.load().paged_attention_prefill(
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["qs"], a["scale"], a["bs"],
        a["hkv"], a["B"], a["hq"], a["d"], a["mb"], a["nb"], a["dtype"], a["mq"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -2),
    (dict(d=96), -3), (dict(bs=12), -3), (dict(hq=30), -3), (dict(B=-1), -3),
    (dict(scale=0.0), -3), (dict(scale=-0.125), -3), (dict(scale=float("nan")), -3),
    (dict(scale=float("inf")), -3),
    (dict(mb=4097), -3),                 # block ids of a sequence live on chip: at most 4096
    (dict(mq=-1), -3), (dict(mq=128 * 16 + 1), -3),   # longer than any context
    (dict(nb=0), -3),
    (dict(out=None), -1), (dict(qs=None), -1), (dict(bt=None), -1),
    (dict(q=FAKE + 8), -7), (dict(out=FAKE + 4), -7), (dict(qs=FAKE + 2), -7),
])
def test_prefill_rejects_before_launch(kw, code):
    assert _prefill(**kw) == code


def test_prefill_empty_is_noop():
    assert _prefill(B=0, out=None, q=None) == 0
    assert _prefill(mq=0, out=None, q=None) == 0


def _prefill_fp8(ks=0.02, vs=0.03, **kw):
    a = dict(out=FAKE, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, cl=FAKE, qs=FAKE, scale=0.125, bs=16,
             hkv=8, B=4, hq=32, d=128, mb=128, nb=1000, dtype=1, mq=512, stream=None)
    a.update(kw)
    return B.load().paged_attention_prefill_fp8(
        a["out"], a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["qs"], a["scale"], ks, vs,
        a["bs"], a["hkv"], a["B"], a["hq"], a["d"], a["mb"], a["nb"], a["dtype"], a["mq"],
        a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ks=0.0), -3), (dict(vs=-1.0), -3), (dict(ks=float("nan")), -3),
    (dict(vs=float("inf")), -3), (dict(ks=1e-45), -3),     # 1 / k_scale overflows
    (dict(dtype=2), -2), (dict(d=96), -3), (dict(mb=4097), -3), (dict(mq=-1), -3),
    (dict(out=None), -1), (dict(kc=None), -1),
    (dict(kc=FAKE + 8), -7), (dict(q=FAKE + 8), -7),
])
def test_prefill_fp8_rejects_before_launch(kw, code):
    assert _prefill_fp8(**kw) == code


def test_prefill_fp8_empty_is_noop():
    assert _prefill_fp8(B=0, out=None, q=None) == 0
    assert _prefill_fp8(mq=0, kc=None, vc=None) == 0
    assert _prefill_fp8(B=0, ks=0.0) == -3     # scales are checked even with no work


@pytest.mark.parametrize("qs,cl,mq,rows,code", [
    ([0, 3, 3, 10], [5, 1, 7], 7, 10, 0),          # an empty chunk in the middle
    ([0, 3, 3, 10], [5, 1, 7], 7, 12, 0),          # q may hold more rows
    ([0, 3, 3, 10], [5, 1, 7], 6, 10, -6),         # chunk of 7 > max_query_len
    ([0, 3, 3, 10], [5, 1, 6], 7, 10, -6),         # chunk longer than its context
    ([1, 3, 3, 10], [5, 1, 7], 7, 10, -6),         # must start at 0
    ([0, 3, 2, 10], [5, 1, 8], 8, 10, -6),         # decreasing
    ([0, 3, 3, 10], [5, 1, 7], 7, 9, -6),          # rows past q
    ([0], [], 0, 0, 0),                            # no sequences
])
def test_validate_prefill(qs, cl, mq, rows, code):
    assert B.validate_prefill(np.array(qs), np.array(cl), mq, rows) == code


def test_validate_prefill_shape_errors():
    lib = B.load()
    assert lib.paged_validate_prefill(None, None, 1, 4, 4) == -1
    assert lib.paged_validate_prefill(FAKE, FAKE, -1, 4, 4) == -3
    with pytest.raises(ValueError):
        B.validate_prefill(np.array([0, 1]), np.array([1, 1]), 1, 1)
