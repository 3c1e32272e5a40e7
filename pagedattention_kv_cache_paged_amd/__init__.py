"""Paged decode attention and paged KV append for AMD Instinct MI355X (gfx950).

The compute lives in libpaged_attn.so (C ABI in include/paged_attn.h);
``binding`` wraps it for torch tensors.  Binding names are imported lazily so
that the input generator (``workloads``) can be used without torch.
"""
_BINDING = ("paged_kv_write", "paged_attention_decode", "paged_kv_write_fp8",
            "paged_attention_decode_fp8", "paged_attention_decode_append",
            "paged_attention_decode_append_noalloc", "paged_attention_decode_shared",
            "workspace_bytes_shared", "validate_shared_prefix",
            "paged_attention_prefill", "paged_attention_prefill_fp8", "paged_copy_blocks",
            "paged_swap_blocks", "BlockPool", "split_waves", "workspace_bytes",
            "validate_metadata", "validate_prefill", "validate_copy_pairs",
            "validate_swap_pairs", "v_shape", "PagedAttentionError", "load")

__all__ = list(_BINDING)


def __getattr__(name):
    if name in _BINDING:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
