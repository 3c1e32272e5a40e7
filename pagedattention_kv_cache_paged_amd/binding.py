"""Thin Python binding of libpaged_attn.so (include/paged_attn.h).

Argument marshalling only: every step of the path runs in the HIP kernels.
PyTorch supplies device memory and the current stream.  torch is imported
before the library is loaded so that the library binds to the same HIP
runtime torch uses; the loader checks that only one HIP runtime is mapped.
There is no CPU fallback: a missing or unloadable library raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpaged_attn.so")
ABI_VERSION = 9  # the argument lists and layouts below are those of this version

PA_F16, PA_BF16 = 0, 1
PA_OK = 0
_ERR_SHAPE = {-2, -3, -7, -8}
SCRATCH_BYTES = 16 << 20  # PA_SCRATCH_BYTES: the no-allocation step's fixed workspace

_DTYPES = {torch.float16: PA_F16, torch.bfloat16: PA_BF16}


class PagedAttentionError(RuntimeError):
    """A call into libpaged_attn returned an error code."""

    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn}: {text} (code {code})")
        self.code = code


_lib = None


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process."""
    with open("/proc/self/maps") as f:
        return sorted({line.split()[-1] for line in f if "libamdhip64" in line})


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m pagedattention_kv_cache_paged_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes loaded: {runtimes}")
    p, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_float, ctypes.c_size_t)
    lib.pa_abi_version.restype = ctypes.c_int
    lib.pa_abi_version.argtypes = []
    if lib.pa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.pa_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild the library")
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_kv_write.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64, i32, p]
    lib.paged_attention_split_waves.restype = i32
    lib.paged_attention_split_waves.argtypes = [i32, i32, i32, i32, i32]
    lib.paged_attention_workspace_bytes.restype = sz
    lib.paged_attention_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    dec = [p, p, p, p, p, p, f32, i32, i32, i32, i32, i32, i32, i64, i32]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode.argtypes = dec + [p, sz, p]
    lib.paged_attention_decode_ex.restype = ctypes.c_int
    lib.paged_attention_decode_ex.argtypes = dec + [i32, p, sz, p]
    lib.paged_attention_decode_stages.restype = ctypes.c_int
    lib.paged_attention_decode_stages.argtypes = dec + [i32, p, sz, i32, p]
    lib.paged_kv_write_fp8.restype = ctypes.c_int
    lib.paged_kv_write_fp8.argtypes = [p, p, p, p, p, i64, i32, i32, i32, i64, i32, f32, f32, p]
    lib.paged_attention_decode_fp8.restype = ctypes.c_int
    lib.paged_attention_decode_fp8.argtypes = [p, p, p, p, p, p, f32, f32, f32, i32, i32, i32,
                                               i32, i32, i32, i64, i32, i32, p, sz, i32, p]
    app = [p, p, p, p, p, p, p, p, f32, f32, f32, i32, i32, i32, i32, i32, i32, i64, i32, i32,
           i32, p, sz]
    lib.paged_attention_decode_append.restype = ctypes.c_int
    lib.paged_attention_decode_append.argtypes = app + [p]
    lib.paged_attention_decode_append_stages.restype = ctypes.c_int
    lib.paged_attention_decode_append_stages.argtypes = app + [i32, p]
    lib.paged_attention_decode_append_noalloc.restype = ctypes.c_int
    lib.paged_attention_decode_append_noalloc.argtypes = app[:-2] + [p]
    lib.paged_attention_decode_shared.restype = ctypes.c_int
    lib.paged_attention_decode_shared.argtypes = app[:-3] + [i32, i32, p, sz, i32, p]
    lib.paged_attention_workspace_bytes_shared.restype = sz
    lib.paged_attention_workspace_bytes_shared.argtypes = [i32, i32, i32, i32, i32, i32, i32,
                                                           i32]
    lib.paged_validate_shared_prefix.restype = ctypes.c_int
    lib.paged_validate_shared_prefix.argtypes = [p, p, i32, i32, i32, i32, i32]
    lib.paged_attention_prefill.restype = ctypes.c_int
    lib.paged_attention_prefill.argtypes = [p, p, p, p, p, p, p, f32, i32, i32, i32, i32, i32,
                                            i32, i64, i32, i32, p]
    lib.paged_attention_prefill_fp8.restype = ctypes.c_int
    lib.paged_attention_prefill_fp8.argtypes = [p, p, p, p, p, p, p, f32, f32, f32, i32, i32,
                                                i32, i32, i32, i32, i64, i32, i32, p]
    lib.pa_pool_create.restype = ctypes.c_int
    lib.pa_pool_create.argtypes = [i64, p, ctypes.POINTER(p)]
    lib.pa_pool_destroy.restype = None
    lib.pa_pool_destroy.argtypes = [p]
    for fn in ("pa_pool_num_blocks", "pa_pool_num_free"):
        getattr(lib, fn).restype = i64
        getattr(lib, fn).argtypes = [p]
    lib.pa_pool_alloc.restype = i64
    lib.pa_pool_alloc.argtypes = [p]
    for fn in ("pa_pool_incref", "pa_pool_decref"):
        getattr(lib, fn).restype = ctypes.c_int
        getattr(lib, fn).argtypes = [p, i64]
    lib.pa_pool_refcount.restype = i32
    lib.pa_pool_refcount.argtypes = [p, i64]
    lib.pa_pool_cow.restype = ctypes.c_int
    lib.pa_pool_cow.argtypes = [p, i64, ctypes.POINTER(i64), ctypes.POINTER(i32)]
    lib.paged_copy_blocks.restype = ctypes.c_int
    lib.paged_copy_blocks.argtypes = [p, p, p, i64, i32, i32, i32, i64, i32, p]
    lib.paged_swap_blocks.restype = ctypes.c_int
    lib.paged_swap_blocks.argtypes = [p, p, i64, p, p, i64, p, i64, i32, i32, i32, i32, p]
    lib.paged_validate_swap_pairs.restype = ctypes.c_int
    lib.paged_validate_swap_pairs.argtypes = [p, i64, i64, i64]
    lib.paged_validate_copy_pairs.restype = ctypes.c_int
    lib.paged_validate_copy_pairs.argtypes = [p, i64, i64]
    lib.paged_validate_metadata.restype = ctypes.c_int
    lib.paged_validate_metadata.argtypes = [p, p, i32, i32, i32, i64, p, i64]
    lib.paged_validate_prefill.restype = ctypes.c_int
    lib.paged_validate_prefill.argtypes = [p, p, i32, i32, i64]
    _lib = lib
    return lib


def v_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int) -> tuple:
    """Shape of a V cache: each (block, KV head) slice holds block_size / 4
    groups of [head_dim][4] (the four positions of a group adjacent per
    dimension)."""
    return (num_blocks, num_kv_heads, block_size // 4, head_dim, 4)


def _check(fn: str, code: int):
    if code != PA_OK:
        text = load().pa_strerror(code).decode()
        if code in _ERR_SHAPE:
            raise ValueError(f"{fn}: {text} (code {code})")
        raise PagedAttentionError(fn, code, text)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")
    return _DTYPES[t.dtype]


def _dev(*ts):
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"expected torch tensors on the GPU, got {type(t).__name__}")
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def split_waves(num_seqs: int, num_kv_heads: int, max_blocks_per_seq: int, block_size: int,
                partition_tokens: int = 0) -> int:
    """Wavefronts per KV head that the decode splits the tiles over."""
    return int(load().paged_attention_split_waves(num_seqs, num_kv_heads, max_blocks_per_seq,
                                                  block_size, partition_tokens))


def workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                    block_size, partition_tokens: int = 0) -> int:
    return int(load().paged_attention_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                                       head_dim, max_blocks_per_seq,
                                                       block_size, partition_tokens))


_workspaces = {}


def workspace(dev, nbytes: int) -> Optional[torch.Tensor]:
    """A cached uint8 device buffer of at least nbytes (grown on demand), one
    per (device, stream): the decode writes its partial results there and
    reads them back in a second launch on the same stream, so calls on
    different streams must not share a buffer.  The buffer is allocated while
    that stream is current, so torch's allocator orders its reuse after the
    stream's queued work when a larger one replaces it."""
    if nbytes == 0:
        return None
    stream = torch.cuda.current_stream(dev)
    key = (dev.type, dev.index, stream.cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(stream):
            ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def paged_kv_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Scatter k, v [T, Hkv, D] into k_cache [N, Hkv, bs, D] and
    v_cache [N, Hkv, bs/4, D, 4] at slot_mapping (int64 [T])."""
    dev = _dev(k, v, slot_mapping, k_cache, v_cache)
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must be [num_tokens, num_kv_heads, head_dim]")
    T, hkv, d = k.shape
    if k_cache.dim() != 4 or k_cache.shape[1] != hkv or k_cache.shape[3] != d:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, _, bs, _ = k_cache.shape
    if tuple(v_cache.shape) != v_shape(nb, hkv, bs, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    dt = _dtype(k)
    if v.dtype != k.dtype or k_cache.dtype != k.dtype or v_cache.dtype != k.dtype:
        raise ValueError("k, v and the caches must share one dtype")
    rc = load().paged_kv_write(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                               k_cache.data_ptr(), v_cache.data_ptr(), T, hkv, d, bs, nb,
                               dt, _stream(dev))
    _check("paged_kv_write", rc)


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: float, block_size: int,
                           num_kv_heads: int, partition_tokens: int = 0,
                           stages: int = 3,
                           workspace_tensor: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[s, h] = softmax(scale * q[s, h] K^T) V over the paged context of
    sequence s.  q, out [B, Hq, D]; block_tables int32 [B, max_blocks];
    context_lens int32 [B].  Returns out."""
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_heads, head_dim]")
    B, hq, d = q.shape
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (num_kv_heads, block_size, d):
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb = k_cache.shape[0]
    if tuple(v_cache.shape) != v_shape(nb, num_kv_heads, block_size, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    dt = _dtype(q)
    if out.dtype != q.dtype or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, out and the caches must share one dtype")
    mb = block_tables.shape[1]
    need = workspace_bytes(B, hq, num_kv_heads, d, mb, block_size, partition_tokens)
    ws = workspace_tensor if workspace_tensor is not None else workspace(dev, need)
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    rc = load().paged_attention_decode_stages(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), block_size,
        num_kv_heads, B, hq, d, mb, nb, dt, partition_tokens, ws_ptr, ws_len, stages,
        _stream(dev))
    _check("paged_attention_decode", rc)
    return out


def validate_metadata(block_tables, context_lens, block_size: int, num_blocks: int,
                      slot_mapping=None) -> int:
    """Host check of tables, lengths and slots (numpy or CPU tensors);
    returns the library's code (0 = valid)."""
    import numpy as np
    bt = np.ascontiguousarray(np.asarray(block_tables), dtype=np.int32)
    cl = np.ascontiguousarray(np.asarray(context_lens), dtype=np.int32)
    sm = None if slot_mapping is None else np.ascontiguousarray(np.asarray(slot_mapping),
                                                                dtype=np.int64)
    return int(load().paged_validate_metadata(
        bt.ctypes.data, cl.ctypes.data, cl.size, bt.shape[1], block_size, num_blocks,
        None if sm is None else sm.ctypes.data, 0 if sm is None else sm.size))


def validate_prefill(query_start, context_lens, max_query_len: int, total_rows: int) -> int:
    """Host check of chunked-prefill offsets against the context lengths
    (numpy or CPU tensors); returns the library's code (0 = valid)."""
    import numpy as np
    qs = np.ascontiguousarray(np.asarray(query_start), dtype=np.int32)
    cl = np.ascontiguousarray(np.asarray(context_lens), dtype=np.int32)
    if qs.size != cl.size + 1:
        raise ValueError("query_start must hold num_seqs + 1 offsets")
    return int(load().paged_validate_prefill(qs.ctypes.data, cl.ctypes.data, cl.size,
                                             max_query_len, total_rows))


# ---- FP8 (E4M3) caches -----------------------------------------------------

def paged_kv_write_fp8(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor,
                       k_cache: torch.Tensor, v_cache: torch.Tensor, k_scale: float,
                       v_scale: float) -> None:
    """Quantise k, v [T, Hkv, D] (fp16 / bf16) into E4M3 caches: uint8
    k_cache [N, Hkv, bs, D] and v_cache [N, Hkv, bs/4, D, 4], at slot_mapping."""
    dev = _dev(k, v, slot_mapping, k_cache, v_cache)
    if k.dim() != 3 or v.shape != k.shape:
        raise ValueError("k and v must be [num_tokens, num_kv_heads, head_dim]")
    T, hkv, d = k.shape
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("FP8 caches are uint8 tensors of E4M3 codes")
    if k_cache.dim() != 4 or k_cache.shape[1] != hkv or k_cache.shape[3] != d:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, _, bs, _ = k_cache.shape
    if tuple(v_cache.shape) != v_shape(nb, hkv, bs, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be int64 [num_tokens]")
    dt = _dtype(k)
    if v.dtype != k.dtype:
        raise ValueError("k and v must share one dtype")
    rc = load().paged_kv_write_fp8(k.data_ptr(), v.data_ptr(), slot_mapping.data_ptr(),
                                   k_cache.data_ptr(), v_cache.data_ptr(), T, hkv, d, bs, nb,
                                   dt, float(k_scale), float(v_scale), _stream(dev))
    _check("paged_kv_write_fp8", rc)


def paged_attention_decode_fp8(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                               v_cache: torch.Tensor, block_tables: torch.Tensor,
                               context_lens: torch.Tensor, scale: float, k_scale: float,
                               v_scale: float, block_size: int, num_kv_heads: int,
                               partition_tokens: int = 0, stages: int = 3,
                               workspace_tensor: Optional[torch.Tensor] = None) -> torch.Tensor:
    """paged_attention_decode over E4M3 caches (uint8 tensors, layouts as
    for the 16-bit caches) with K = code * k_scale, V = code * v_scale."""
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_heads, head_dim]")
    B, hq, d = q.shape
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("FP8 caches are uint8 tensors of E4M3 codes")
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (num_kv_heads, block_size, d):
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb = k_cache.shape[0]
    if tuple(v_cache.shape) != v_shape(nb, num_kv_heads, block_size, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    dt = _dtype(q)
    if out.dtype != q.dtype:
        raise ValueError("q and out must share one dtype")
    mb = block_tables.shape[1]
    need = workspace_bytes(B, hq, num_kv_heads, d, mb, block_size, partition_tokens)
    ws = workspace_tensor if workspace_tensor is not None else workspace(dev, need)
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    rc = load().paged_attention_decode_fp8(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), float(k_scale),
        float(v_scale), block_size, num_kv_heads, B, hq, d, mb, nb, dt, partition_tokens,
        ws_ptr, ws_len, stages, _stream(dev))
    _check("paged_attention_decode_fp8", rc)
    return out



# ---- decode step with the append fused in ---------------------------------

def _append_shapes(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                   block_size, num_kv_heads, k_scale, v_scale):
    """Checks of the fused step's tensors; returns (dev, B, hq, d, mb, nb, dt, fp8)."""
    dev = _dev(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [num_seqs, num_heads, head_dim]")
    B, hq, d = q.shape
    if tuple(k_new.shape) != (B, num_kv_heads, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (num_kv_heads, block_size, d):
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb = k_cache.shape[0]
    if tuple(v_cache.shape) != v_shape(nb, num_kv_heads, block_size, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or tuple(context_lens.shape) != (B,):
        raise ValueError("context_lens must be int32 [num_seqs]")
    dt = _dtype(q)
    if out.dtype != q.dtype or k_new.dtype != q.dtype or v_new.dtype != q.dtype:
        raise ValueError("q, out, k_new and v_new must share one dtype")
    fp8 = k_cache.dtype == torch.uint8
    if fp8:
        if v_cache.dtype != torch.uint8 or k_scale is None or v_scale is None:
            raise ValueError("E4M3 caches: both uint8, with k_scale and v_scale")
    elif k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("16-bit caches must share q's dtype")
    return dev, B, hq, d, block_tables.shape[1], nb, dt, fp8


def paged_attention_decode_append(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                                  v_new: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, block_size: int,
                                  num_kv_heads: int, k_scale: Optional[float] = None,
                                  v_scale: Optional[float] = None, partition_tokens: int = 0,
                                  workspace_tensor: Optional[torch.Tensor] = None,
                                  stages: int = 3) -> torch.Tensor:
    """Store each sequence's new token (k_new, v_new [B, Hkv, D]) at context
    position L-1 of its block table, then decode over all L tokens.  uint8
    caches hold E4M3 codes and need k_scale, v_scale; 16-bit caches share
    q's dtype.  stages: 1 split pass (with the stores), 2 merge, 3 both.
    Returns out."""
    dev, B, hq, d, mb, nb, dt, fp8 = _append_shapes(out, q, k_new, v_new, k_cache, v_cache,
                                                    block_tables, context_lens, block_size,
                                                    num_kv_heads, k_scale, v_scale)
    need = workspace_bytes(B, hq, num_kv_heads, d, mb, block_size, partition_tokens)
    ws = workspace_tensor if workspace_tensor is not None else workspace(dev, need)
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    rc = load().paged_attention_decode_append_stages(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
        float(k_scale or 1.0), float(v_scale or 1.0), block_size, num_kv_heads, B, hq, d, mb,
        nb, dt, 1 if fp8 else 0, partition_tokens, ws_ptr, ws_len, stages, _stream(dev))
    _check("paged_attention_decode_append", rc)
    return out


def paged_attention_decode_append_noalloc(out: torch.Tensor, q: torch.Tensor,
                                          k_new: torch.Tensor, v_new: torch.Tensor,
                                          k_cache: torch.Tensor, v_cache: torch.Tensor,
                                          block_tables: torch.Tensor,
                                          context_lens: torch.Tensor, scale: float,
                                          block_size: int, num_kv_heads: int,
                                          k_scale: Optional[float] = None,
                                          v_scale: Optional[float] = None,
                                          partition_tokens: int = 0) -> torch.Tensor:
    """paged_attention_decode_append with the library's fixed per-GPU
    scratch array as its workspace: allocates nothing.  Calls that overlap on
    one GPU race.  Sizes needing more than SCRATCH_BYTES raise ValueError."""
    dev, B, hq, d, mb, nb, dt, fp8 = _append_shapes(out, q, k_new, v_new, k_cache, v_cache,
                                                    block_tables, context_lens, block_size,
                                                    num_kv_heads, k_scale, v_scale)
    rc = load().paged_attention_decode_append_noalloc(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
        float(k_scale or 1.0), float(v_scale or 1.0), block_size, num_kv_heads, B, hq, d, mb,
        nb, dt, 1 if fp8 else 0, partition_tokens, _stream(dev))
    _check("paged_attention_decode_append_noalloc", rc)
    return out


# ---- decode with a prefix shared by the whole batch ---------------------------

def workspace_bytes_shared(num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                           block_size, shared_blocks, partition_tokens: int = 0) -> int:
    return int(load().paged_attention_workspace_bytes_shared(
        num_seqs, num_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
        shared_blocks, partition_tokens))


def paged_attention_decode_shared(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                  v_cache: torch.Tensor, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, scale: float, block_size: int,
                                  num_kv_heads: int, shared_blocks: int,
                                  k_new: Optional[torch.Tensor] = None,
                                  v_new: Optional[torch.Tensor] = None,
                                  k_scale: Optional[float] = None,
                                  v_scale: Optional[float] = None, partition_tokens: int = 0,
                                  stages: int = 3,
                                  workspace_tensor: Optional[torch.Tensor] = None
                                  ) -> torch.Tensor:
    """Decode (k_new, v_new None) or the fused step (both given) when every
    sequence's first shared_blocks table entries are the same blocks and
    every context covers them: the prefix is streamed once per group of
    sequences.  uint8 caches hold E4M3 codes (k_scale, v_scale).  Returns out."""
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    append = k_new is not None
    kn = k_new if append else q.new_empty((q.shape[0], num_kv_heads, q.shape[2]))
    vn = v_new if append else kn
    dev, B, hq, d, mb, nb, dt, fp8 = _append_shapes(out, q, kn, vn, k_cache, v_cache,
                                                    block_tables, context_lens, block_size,
                                                    num_kv_heads, k_scale, v_scale)
    need = workspace_bytes_shared(B, hq, num_kv_heads, d, mb, block_size, shared_blocks,
                                  partition_tokens)
    ws = workspace_tensor if workspace_tensor is not None else workspace(dev, need)
    ws_ptr = ws.data_ptr() if ws is not None else None
    ws_len = ws.numel() * ws.element_size() if ws is not None else 0
    rc = load().paged_attention_decode_shared(
        out.data_ptr(), q.data_ptr(), kn.data_ptr() if append else None,
        vn.data_ptr() if append else None, k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), float(k_scale or 1.0),
        float(v_scale or 1.0), block_size, num_kv_heads, B, hq, d, mb, nb, dt, 1 if fp8 else 0,
        int(shared_blocks), partition_tokens, ws_ptr, ws_len, stages, _stream(dev))
    _check("paged_attention_decode_shared", rc)
    return out


def validate_shared_prefix(block_tables, context_lens, block_size: int, shared_blocks: int,
                           append: bool = False) -> int:
    """Host check of the shared-prefix contract (numpy or CPU tensors);
    returns the library's code (0 = valid)."""
    import numpy as np
    bt = np.ascontiguousarray(np.asarray(block_tables), dtype=np.int32)
    cl = np.ascontiguousarray(np.asarray(context_lens), dtype=np.int32)
    return int(load().paged_validate_shared_prefix(bt.ctypes.data, cl.ctypes.data, cl.size,
                                                   bt.shape[1], block_size, shared_blocks,
                                                   1 if append else 0))


# ---- block pool and copy-on-write (include/paged_blocks.h) ------------------

class BlockPool:
    """Reference-counted pool of physical block ids (host object of the
    library).  alloc() returns -1 when the pool is exhausted."""

    def __init__(self, num_blocks: int, order=None):
        import numpy as np
        lib = load()
        self._order = None if order is None else np.ascontiguousarray(order, dtype=np.int64)
        h = ctypes.c_void_p()
        _check("pa_pool_create", lib.pa_pool_create(
            num_blocks, None if self._order is None else self._order.ctypes.data,
            ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            load().pa_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return int(load().pa_pool_num_blocks(self._h))

    @property
    def num_free(self) -> int:
        return int(load().pa_pool_num_free(self._h))

    def alloc(self) -> int:
        return int(load().pa_pool_alloc(self._h))

    def incref(self, block: int) -> None:
        _check("pa_pool_incref", load().pa_pool_incref(self._h, block))

    def decref(self, block: int) -> None:
        _check("pa_pool_decref", load().pa_pool_decref(self._h, block))

    def refcount(self, block: int) -> int:
        return int(load().pa_pool_refcount(self._h, block))

    def cow(self, block: int):
        """(dst, copy): the block to write into and whether block -> dst
        must be copied first."""
        dst, copy = ctypes.c_int64(), ctypes.c_int32()
        _check("pa_pool_cow", load().pa_pool_cow(self._h, block, ctypes.byref(dst),
                                                 ctypes.byref(copy)))
        return int(dst.value), bool(copy.value)


def paged_copy_blocks(pairs: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor
                      ) -> None:
    """Block pairs[i, 1] of both caches becomes a copy of block pairs[i, 0]
    (int64 [n, 2] on the caches' device; negative ids skipped).  16-bit or
    uint8 (E4M3) caches in the layouts of paged_kv_write."""
    dev = _dev(pairs, k_cache, v_cache)
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int64 [num_pairs, 2]")
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, d = k_cache.shape
    if tuple(v_cache.shape) != v_shape(nb, hkv, bs, d) or v_cache.dtype != k_cache.dtype:
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4], "
                         "k_cache's dtype")
    rc = load().paged_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), pairs.data_ptr(),
                                  pairs.shape[0], hkv, d, bs, nb, k_cache.element_size(),
                                  _stream(dev))
    _check("paged_copy_blocks", rc)


def validate_copy_pairs(pairs, num_blocks: int) -> int:
    import numpy as np
    pr = np.ascontiguousarray(np.asarray(pairs), dtype=np.int64).reshape(-1, 2)
    return int(load().paged_validate_copy_pairs(pr.ctypes.data, pr.shape[0], num_blocks))


def paged_swap_blocks(pairs: torch.Tensor, dst_k: torch.Tensor, dst_v: torch.Tensor,
                      src_k: torch.Tensor, src_v: torch.Tensor,
                      stream_device: Optional[torch.device] = None) -> None:
    """Block pairs[i, 1] of (dst_k, dst_v) becomes block pairs[i, 0] of
    (src_k, src_v): device caches <-> a pinned host pool of the same layout
    (swap-out / swap-in).  pairs: int64 [n, 2] on the device or pinned.
    Runs on the current stream of the GPU involved."""
    for t in (dst_k, dst_v, src_k, src_v, pairs):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device.type == "cpu" and not t.is_pinned():
            raise ValueError("host tensors must be pinned (pin_memory=True)")
    dev = stream_device or next((t.device for t in (dst_k, src_k, pairs)
                                 if t.device.type == "cuda"), None)
    if dev is None:
        raise ValueError("one side of the swap must be a GPU tensor")
    if pairs.dtype != torch.int64 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int64 [num_pairs, 2]")
    nd, hkv, bs, d = dst_k.shape
    ns = src_k.shape[0]
    if (tuple(src_k.shape[1:]) != (hkv, bs, d) or
            tuple(dst_v.shape) != v_shape(nd, hkv, bs, d) or
            tuple(src_v.shape) != v_shape(ns, hkv, bs, d)):
        raise ValueError("pools must share the cache layouts and sizes per block")
    if len({t.dtype for t in (dst_k, dst_v, src_k, src_v)}) != 1:
        raise ValueError("pools must share one element type")
    rc = load().paged_swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), nd, src_k.data_ptr(),
                                  src_v.data_ptr(), ns, pairs.data_ptr(), pairs.shape[0], hkv,
                                  d, bs, dst_k.element_size(), _stream(dev))
    _check("paged_swap_blocks", rc)


def validate_swap_pairs(pairs, src_num_blocks: int, dst_num_blocks: int) -> int:
    import numpy as np
    pr = np.ascontiguousarray(np.asarray(pairs), dtype=np.int64).reshape(-1, 2)
    return int(load().paged_validate_swap_pairs(pr.ctypes.data, pr.shape[0], src_num_blocks,
                                                dst_num_blocks))


# ---- paged (chunked) prefill -------------------------------------------------

def _prefill_shapes(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                    block_size, num_kv_heads):
    dev = _dev(out, q, k_cache, v_cache, block_tables, context_lens, query_start)
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be [rows, num_heads, head_dim]")
    rows, hq, d = q.shape
    B = context_lens.shape[0]
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (num_kv_heads, block_size, d):
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, block_size, head_dim]")
    nb = k_cache.shape[0]
    if tuple(v_cache.shape) != v_shape(nb, num_kv_heads, block_size, d):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size / 4, head_dim, 4]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [num_seqs, max_blocks_per_seq]")
    if context_lens.dtype != torch.int32 or context_lens.dim() != 1:
        raise ValueError("context_lens must be int32 [num_seqs]")
    if query_start.dtype != torch.int32 or tuple(query_start.shape) != (B + 1,):
        raise ValueError("query_start must be int32 [num_seqs + 1]")
    dt = _dtype(q)
    if out.dtype != q.dtype:
        raise ValueError("q and out must share one dtype")
    return dev, B, hq, d, nb, dt


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                            v_cache: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, query_start: torch.Tensor,
                            scale: float, block_size: int, num_kv_heads: int,
                            max_query_len: int) -> torch.Tensor:
    """Rows query_start[s] .. query_start[s+1]-1 of q / out ([rows, Hq, D])
    are sequence s's last positions; each attends causally over the paged
    context up to its own position.  Returns out."""
    dev, B, hq, d, nb, dt = _prefill_shapes(out, q, k_cache, v_cache, block_tables,
                                            context_lens, query_start, block_size,
                                            num_kv_heads)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q, out and the caches must share one dtype")
    rc = load().paged_attention_prefill(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), float(scale),
        block_size, num_kv_heads, B, hq, d, block_tables.shape[1], nb, dt, int(max_query_len),
        _stream(dev))
    _check("paged_attention_prefill", rc)
    return out


def paged_attention_prefill_fp8(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                v_cache: torch.Tensor, block_tables: torch.Tensor,
                                context_lens: torch.Tensor, query_start: torch.Tensor,
                                scale: float, k_scale: float, v_scale: float,
                                block_size: int, num_kv_heads: int,
                                max_query_len: int) -> torch.Tensor:
    """paged_attention_prefill over E4M3 caches (uint8 tensors, layouts as
    for the 16-bit caches) with K = code * k_scale, V = code * v_scale."""
    dev, B, hq, d, nb, dt = _prefill_shapes(out, q, k_cache, v_cache, block_tables,
                                            context_lens, query_start, block_size,
                                            num_kv_heads)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("FP8 caches are uint8 tensors of E4M3 codes")
    rc = load().paged_attention_prefill_fp8(
        out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(), float(scale),
        float(k_scale), float(v_scale), block_size, num_kv_heads, B, hq, d,
        block_tables.shape[1], nb, dt, int(max_query_len), _stream(dev))
    _check("paged_attention_prefill_fp8", rc)
    return out
