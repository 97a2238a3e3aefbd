"""ctypes view of libpagedattn.so (the C ABI in include/pagedattn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

PA_OK = 0
PA_ERR_NULL = 1
PA_ERR_SHAPE = 2
PA_ERR_UNSUPPORTED = 3
PA_ERR_ALIGN = 4
PA_ERR_WORKSPACE = 5
PA_ERR_HIP = 6
PA_ERR_SCRATCH_LIMIT = 7
PA_ERR_PRECONDITION = 8
PA_DTYPE_F32 = 0
PA_DTYPE_BF16 = 1

SIZE_MAX = ctypes.c_size_t(-1).value
PA_NOALLOC_SCRATCH_BYTES = 32 << 20


class DecodeDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p * 2),
    ]


class PrefillDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("stream", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p * 2),
    ]


class CacheDims(ctypes.Structure):
    _fields_ = [
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
    ]


class RopeDims(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("rot_dim", ctypes.c_int32),
        ("max_position", ctypes.c_int32),
        ("is_neox", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class CopyDims(ctypes.Structure):
    _fields_ = [
        ("num_pairs", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("src_num_blocks", ctypes.c_int32),
        ("dst_num_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
    ]


# name -> (restype, argtypes); every symbol include/pagedattn.h declares
SIGNATURES = {
    "paged_attention_decode": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_alibi": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_step": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_partition_tokens": (ctypes.c_int32, [
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_shared_prefix": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_shared_prefix_step": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_decode_shared_prefix_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
    "paged_attention_prefill": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(PrefillDims)]),
    "paged_attention_prefill_alibi": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(PrefillDims)]),
    "paged_attention_prefill_step": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.POINTER(PrefillDims)]),
    "paged_attention_prefill_workspace_bytes": (ctypes.c_size_t, [
        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(PrefillDims)]),
    "paged_attention_prefill_partition_tokens": (ctypes.c_int32, [
        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(PrefillDims)]),
    "reshape_and_cache": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.POINTER(CacheDims)]),
    "reshape_and_cache_rope": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(RopeDims),
        ctypes.POINTER(CacheDims)]),
    "copy_blocks": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.POINTER(CopyDims)]),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_hbm_read_probe": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "pa_hbm_read_probe_sink_bytes": (ctypes.c_size_t, []),
    "paged_attention_decode_read_probe": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(DecodeDims)]),
}

_lib = None


def load() -> ctypes.CDLL:
    """The loaded library, with argument and return types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m paged_kv_cache_457_amd.build` "
            "(or __graft_entry__.build()) first")
    # torch ships its own HIP runtime with the same soname as ROCm's.  Load
    # torch first so that this library binds to the runtime torch already
    # uses (one runtime per process; device pointers and streams are shared).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    _lib = bind(ctypes.CDLL(LIB_PATH))
    return _lib


def bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Set the argument and return types of every declared entry point on
    a loaded library."""
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def status_string(rc: int) -> str:
    return load().pa_status_string(rc).decode()
