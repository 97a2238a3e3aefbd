"""libpagedattn: paged decode attention and the KV-cache write on MI355X.

The compute path is the HIP library ``libpagedattn.so`` (C ABI in
``include/pagedattn.h``); ``binding`` marshals torch tensors to it.  Import
of the tensor functions is lazy so that ``workloads`` (input generation,
NumPy only) can be used without torch or a built library.
"""
__all__ = [
    "paged_attention_decode", "paged_attention_decode_step", "paged_attention_decode_shared_prefix",
    "paged_attention_decode_shared_prefix_step", "paged_attention_decode_noalloc",
    "paged_attention_decode_read_probe", "paged_attention_prefill", "paged_attention_prefill_step",
    "reshape_and_cache", "reshape_and_cache_rope", "copy_blocks",
    "paged_attention_decode_shared_prefix_workspace_bytes",
    "paged_attention_decode_workspace_bytes", "paged_attention_decode_partition_tokens",
    "paged_attention_prefill_workspace_bytes", "paged_attention_prefill_partition_tokens",
    "hbm_read_probe", "PagedAttnError",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
