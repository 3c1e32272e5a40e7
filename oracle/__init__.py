"""fp64 CPU oracle for paged decode attention and the paged KV append.

TEST INFRASTRUCTURE ONLY: this package may be imported by ``tests/``, by the
package's ``smoke()`` check and by the benchmark's CPU-baseline leg, and by
nothing else.  It shares no code with the HIP library; the only module both
sides use is the seeded input generator (``workloads``), which holds none of
the attention arithmetic.

The arithmetic lives in ``oracle.c`` (plain C, double precision, compiled with
gcc without fast-math or FMA contraction).  This module only builds that file
and marshals numpy arrays into it.

Storage convention (identical to the library's documented one, implemented
independently in ``oracle.c``):

* K cache ``uint16 [num_blocks, num_kv_heads, block_size, head_dim]``
* V cache ``uint16 [num_blocks, num_kv_heads, block_size // 4, head_dim, 4]``: positions in
  groups of four, the four positions of one dimension adjacent.
* q ``uint16 [num_seqs, num_heads, head_dim]``; k, v ``uint16 [T, num_kv_heads, head_dim]``
* ``dtype`` 0 = IEEE binary16, 1 = bfloat16 (raw bit patterns).
* FP8 caches: uint8 OCP E4M3 codes in the same layouts, standing for
  code * k_scale (K) or code * v_scale (V); the append quantises
  float32(x) * float32(1 / scale) to the nearest code, saturating at +-448.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F16, BF16 = 0, 1
_DTYPE = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}

ERRORS = {
    -1: "bad sizes or dtype",
    -2: "slot out of range or repeated",
    -3: "block table names a block outside the pool",
    -4: "context length exceeds the block table's capacity",
    -5: "normalised weights do not sum to one",
    -6: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", f"{out}.tmp{os.getpid()}", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(f"{out}.tmp{os.getpid()}", out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("PAGED_ORACLE_LIB")  # mutation tests load a planted-mistake build
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
    p = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = dbl
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = dbl
    lib.oracle_kv_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64]
    lib.oracle_kv_write.restype = i32
    common = [p, p, p, p, p, dbl, i32, i32, i32, i32, i32, i32, i64, i32]
    lib.oracle_decode.argtypes = [p] + common
    lib.oracle_decode.restype = i32
    lib.oracle_decode_rows.argtypes = [p, p, i32] + common
    lib.oracle_decode_rows.restype = i32
    lib.oracle_decode_row_partitioned.argtypes = [p] + common + [i32, i32, i32]
    lib.oracle_decode_row_partitioned.restype = i32
    lib.oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_f64.restype = dbl
    lib.oracle_f64_to_e4m3.argtypes = [dbl]
    lib.oracle_f64_to_e4m3.restype = ctypes.c_uint8
    f32 = ctypes.c_float
    lib.oracle_kv_write_fp8.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64, i32, f32, f32]
    lib.oracle_kv_write_fp8.restype = i32
    common8 = [p, p, p, p, p, dbl, i32, i32, i32, i32, i32, i32, i64, i32, dbl, dbl]
    lib.oracle_decode_fp8.argtypes = [p] + common8
    lib.oracle_decode_fp8.restype = i32
    lib.oracle_decode_fp8_rows.argtypes = [p, p, i32] + common8
    lib.oracle_decode_fp8_rows.restype = i32
    lib.oracle_copy_blocks.argtypes = [p, p, p, i64, i32, i32, i32, i64, i32]
    lib.oracle_copy_blocks.restype = i32
    lib.oracle_swap_blocks.argtypes = [p, p, i64, p, p, i64, p, i64, i32, i32, i32, i32]
    lib.oracle_swap_blocks.restype = i32
    lib.oracle_prefill.argtypes = [p, p, p, p, p, p, p, dbl, i32, i32, i32, i32, i32, i32, i64,
                                   i32]
    lib.oracle_prefill.restype = i32
    lib.oracle_prefill_fp8.argtypes = [p, p, p, p, p, p, p, dbl, i32, i32, i32, i32, i32, i32,
                                       i64, i32, dbl, dbl]
    lib.oracle_prefill_fp8.restype = i32
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {ERRORS.get(rc, rc)}")


def dtype_code(dtype) -> int:
    if isinstance(dtype, int):
        return dtype
    return _DTYPE[str(dtype)]


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits))


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits))


def decode_bits(bits: np.ndarray, dtype) -> np.ndarray:
    """Element-wise decode of a uint16 array through the oracle's decoders
    (slow; meant for small arrays in tests)."""
    fn = f16_to_f64 if dtype_code(dtype) == F16 else bf16_to_f64
    flat = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    return np.array([fn(b) for b in flat], dtype=np.float64).reshape(bits.shape)


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def kv_write(k, v, slot_mapping, k_cache, v_cache, block_size: int) -> None:
    """In-place scatter of k/v [T, Hkv, D] into the caches at slot_mapping."""
    k, v = _u16(k), _u16(v)
    slot = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint16 and v_cache.dtype == np.uint16
    T, hkv, d = k.shape
    nb = k_cache.shape[0]
    assert k_cache.shape == (nb, hkv, block_size, d)
    assert v_cache.shape == (nb, hkv, block_size // 4, d, 4)
    rc = _load().oracle_kv_write(_ptr(k), _ptr(v), _ptr(slot), _ptr(k_cache),
                                 _ptr(v_cache), T, hkv, d, block_size, nb)
    _check(rc, "oracle_kv_write")


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, scale,
                 block_size, dtype):
    q = _u16(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    kc, vc = _u16(k_cache), _u16(v_cache)
    B, hq, d = q.shape
    nb, hkv = kc.shape[0], kc.shape[1]
    assert kc.shape == (nb, hkv, block_size, d)
    assert vc.shape == (nb, hkv, block_size // 4, d, 4)
    assert bt.shape[0] == B and cl.shape == (B,)
    keep = (q, bt, cl, kc, vc)
    args = [_ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl), float(scale),
            block_size, hkv, B, hq, d, bt.shape[1], nb, dtype_code(dtype)]
    return keep, args, (B, hq, d)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
           dtype) -> np.ndarray:
    """Full decode attention; returns float64 [B, Hq, D]."""
    keep, args, (B, hq, d) = _decode_args(q, k_cache, v_cache, block_tables,
                                          context_lens, scale, block_size, dtype)
    out = np.zeros((B, hq, d), dtype=np.float64)
    _check(_load().oracle_decode(_ptr(out), *args), "oracle_decode")
    del keep
    return out


def all_rows(num_seqs: int, num_heads: int) -> np.ndarray:
    """Every (seq, head) pair, sequence-major: int32 [num_seqs * num_heads, 2]."""
    s, h = np.meshgrid(np.arange(num_seqs), np.arange(num_heads), indexing="ij")
    return np.ascontiguousarray(np.stack([s.ravel(), h.ravel()], 1), dtype=np.int32)


def host_threads() -> int:
    """Threads for a pooled oracle run: the CPUs this process may use, at
    most 16 (one GPU's share of a GPU host's cores)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pooled(fn, rows, d, threads):
    """fn(out_chunk, rows_chunk) over chunks of rows on a pool of host
    threads; the C oracle runs outside Python's lock, so the chunks run
    concurrently.  Each row is computed exactly as in a single call."""
    out = np.zeros((rows.shape[0], d), dtype=np.float64)
    if threads <= 1 or rows.shape[0] <= 1:
        fn(out, rows)
        return out
    from concurrent.futures import ThreadPoolExecutor
    n = min(rows.shape[0], threads * 8)
    bounds = np.linspace(0, rows.shape[0], n + 1).astype(np.int64)

    def run(i):
        a, b = int(bounds[i]), int(bounds[i + 1])
        if b > a:
            chunk_out = np.zeros((b - a, d), dtype=np.float64)
            fn(chunk_out, np.ascontiguousarray(rows[a:b]))
            out[a:b] = chunk_out
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, range(n)))
    return out


def decode_rows(rows, q, k_cache, v_cache, block_tables, context_lens, scale,
                block_size, dtype, threads: int = 1) -> np.ndarray:
    """Selected (seq, head) rows; returns float64 [len(rows), D].  With
    threads > 1 the rows are shared out over that many host threads."""
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
    keep, args, (_, _, d) = _decode_args(q, k_cache, v_cache, block_tables,
                                         context_lens, scale, block_size, dtype)
    lib = _load()

    def fn(out, rr):
        _check(lib.oracle_decode_rows(_ptr(out), _ptr(rr), rr.shape[0], *args),
               "oracle_decode_rows")
    out = _pooled(fn, rows, d, threads)
    del keep
    return out


def decode_row_partitioned(s, h, part_tokens, q, k_cache, v_cache, block_tables,
                           context_lens, scale, block_size, dtype) -> np.ndarray:
    """One row computed partition by partition and merged by log-sum-exp."""
    keep, args, (_, _, d) = _decode_args(q, k_cache, v_cache, block_tables,
                                         context_lens, scale, block_size, dtype)
    out = np.zeros((d,), dtype=np.float64)
    _check(_load().oracle_decode_row_partitioned(_ptr(out), *args, int(s), int(h),
                                                 int(part_tokens)),
           "oracle_decode_row_partitioned")
    del keep
    return out


# ---- FP8 (E4M3) cache ------------------------------------------------------

FP8_NAN = 0x7F


def e4m3_to_f64(code: int) -> float:
    return _load().oracle_e4m3_to_f64(int(code))


def f64_to_e4m3(y: float) -> int:
    return int(_load().oracle_f64_to_e4m3(float(y)))


def kv_write_fp8(k, v, slot_mapping, k_cache, v_cache, block_size: int, dtype,
                 k_scale: float, v_scale: float) -> None:
    """In-place quantising scatter of 16-bit k/v [T, Hkv, D] into uint8 E4M3
    caches ([N, Hkv, bs, D] and [N, Hkv, bs // 4, D, 4]) at slot_mapping."""
    k, v = _u16(k), _u16(v)
    slot = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == np.uint8 and v_cache.dtype == np.uint8
    T, hkv, d = k.shape
    nb = k_cache.shape[0]
    assert k_cache.shape == (nb, hkv, block_size, d)
    assert v_cache.shape == (nb, hkv, block_size // 4, d, 4)
    rc = _load().oracle_kv_write_fp8(_ptr(k), _ptr(v), _ptr(slot), _ptr(k_cache),
                                     _ptr(v_cache), T, hkv, d, block_size, nb,
                                     dtype_code(dtype), float(k_scale), float(v_scale))
    _check(rc, "oracle_kv_write_fp8")


def _decode_fp8_args(q, k_cache, v_cache, block_tables, context_lens, scale, block_size,
                     q_dtype, k_scale, v_scale):
    q = _u16(q)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    kc = np.ascontiguousarray(k_cache)
    vc = np.ascontiguousarray(v_cache)
    assert kc.dtype == np.uint8 and vc.dtype == np.uint8
    B, hq, d = q.shape
    nb, hkv = kc.shape[0], kc.shape[1]
    assert kc.shape == (nb, hkv, block_size, d)
    assert vc.shape == (nb, hkv, block_size // 4, d, 4)
    keep = (q, bt, cl, kc, vc)
    args = [_ptr(q), _ptr(kc), _ptr(vc), _ptr(bt), _ptr(cl), float(scale), block_size, hkv,
            B, hq, d, bt.shape[1], nb, dtype_code(q_dtype), float(k_scale), float(v_scale)]
    return keep, args, (B, hq, d)


def decode_fp8(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, q_dtype,
               k_scale, v_scale) -> np.ndarray:
    """Decode attention over E4M3 caches; returns float64 [B, Hq, D]."""
    keep, args, (B, hq, d) = _decode_fp8_args(q, k_cache, v_cache, block_tables,
                                              context_lens, scale, block_size, q_dtype,
                                              k_scale, v_scale)
    out = np.zeros((B, hq, d), dtype=np.float64)
    _check(_load().oracle_decode_fp8(_ptr(out), *args), "oracle_decode_fp8")
    del keep
    return out


def decode_fp8_rows(rows, q, k_cache, v_cache, block_tables, context_lens, scale,
                    block_size, q_dtype, k_scale, v_scale, threads: int = 1) -> np.ndarray:
    """Selected (seq, head) rows of decode_fp8; returns float64 [len(rows), D].
    With threads > 1 the rows are shared out over that many host threads."""
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 2)
    keep, args, (_, _, d) = _decode_fp8_args(q, k_cache, v_cache, block_tables, context_lens,
                                             scale, block_size, q_dtype, k_scale, v_scale)
    lib = _load()

    def fn(out, rr):
        _check(lib.oracle_decode_fp8_rows(_ptr(out), _ptr(rr), rr.shape[0], *args),
               "oracle_decode_fp8_rows")
    out = _pooled(fn, rows, d, threads)
    del keep
    return out



def copy_blocks(pairs, k_cache, v_cache, block_size: int) -> None:
    """In-place copy-on-write block copies: for each (src, dst) row of
    pairs (int64 [n, 2]; negative ids skipped), block dst of both caches
    (16-bit bits or uint8 E4M3 codes) becomes block src."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == v_cache.dtype and k_cache.dtype.itemsize in (1, 2)
    nb, hkv, bs, d = k_cache.shape
    assert bs == block_size and v_cache.shape == (nb, hkv, bs // 4, d, 4)
    rc = _load().oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pairs), pairs.shape[0],
                                    hkv, d, bs, nb, k_cache.dtype.itemsize)
    _check(rc, "oracle_copy_blocks")


def swap_blocks(pairs, dst_k, dst_v, src_k, src_v, block_size: int) -> None:
    """Block copies between two pools (swap-out / swap-in): for each (src,
    dst) row of pairs, block dst of (dst_k, dst_v) becomes block src of
    (src_k, src_v); negative ids are skipped."""
    pairs = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    for a in (dst_k, dst_v, src_k, src_v):
        assert a.flags.c_contiguous and a.dtype == dst_k.dtype and a.dtype.itemsize in (1, 2)
    nd, hkv, bs, d = dst_k.shape
    ns = src_k.shape[0]
    assert bs == block_size and src_k.shape[1:] == dst_k.shape[1:]
    assert dst_v.shape == (nd, hkv, bs // 4, d, 4) and src_v.shape == (ns, hkv, bs // 4, d, 4)
    rc = _load().oracle_swap_blocks(_ptr(dst_k), _ptr(dst_v), nd, _ptr(src_k), _ptr(src_v), ns,
                                    _ptr(pairs), pairs.shape[0], hkv, d, bs,
                                    dst_k.dtype.itemsize)
    _check(rc, "oracle_swap_blocks")


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
            block_size: int, dtype) -> np.ndarray:
    """Chunked-prefill attention: q [total_q, Hq, D] bits, rows
    query_start[s] .. query_start[s+1]-1 are sequence s's last positions
    L-n .. L-1, each attending causally over positions 0 .. its own.
    Returns float64 [total_q, Hq, D]."""
    q = _u16(q)
    k_cache, v_cache = _u16(k_cache), _u16(v_cache)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    total, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    assert bs == block_size and qs.size == cl.size + 1 and qs[-1] == total
    out = np.zeros((total, hq, d), dtype=np.float64)
    _check(_load().oracle_prefill(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt),
                                  _ptr(cl), _ptr(qs), float(scale), bs, hkv, cl.size, hq, d,
                                  bt.shape[1], nb, dtype_code(dtype)), "oracle_prefill")
    return out


def prefill_fp8(q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
                block_size: int, q_dtype, k_scale: float, v_scale: float) -> np.ndarray:
    """Chunked prefill over E4M3 caches (uint8 codes; K = code * k_scale,
    V = code * v_scale); q [total_q, Hq, D] bits of q_dtype.  Returns float64
    [total_q, Hq, D]."""
    q = _u16(q)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint8)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint8)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    total, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    assert bs == block_size and qs.size == cl.size + 1 and qs[-1] == total
    out = np.zeros((total, hq, d), dtype=np.float64)
    _check(_load().oracle_prefill_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(bt), _ptr(cl), _ptr(qs), float(scale), bs, hkv,
                                      cl.size, hq, d, bt.shape[1], nb, dtype_code(q_dtype),
                                      float(k_scale), float(v_scale)), "oracle_prefill_fp8")
    return out
