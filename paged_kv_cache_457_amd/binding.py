"""Torch-tensor front end of libpagedattn (argument marshalling only).

Every function here checks devices, dtypes and contiguity, reads shapes off
the tensors, passes raw device pointers and torch's current HIP stream to
the C ABI, and raises on a nonzero status.  All arithmetic runs in the HIP
kernels; nothing here computes attention or touches tensor contents.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.PA_DTYPE_F32, torch.bfloat16: _lib.PA_DTYPE_BF16}


class PagedAttnError(RuntimeError):
    def __init__(self, rc: int, where: str):
        self.rc = rc
        super().__init__(f"{where}: {_lib.status_string(rc)}")


def _check(rc: int, where: str) -> None:
    if rc != _lib.PA_OK:
        raise PagedAttnError(rc, where)


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream_ptr(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _event_ptr(ev) -> Optional[int]:
    """A raw hipEvent_t from a torch.cuda.Event (already recorded once, so
    that it exists) or an int handle; None for no event."""
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    handle = getattr(ev, "cuda_event", 0)
    if not handle:
        raise ValueError("record a torch.cuda.Event once before passing it as a timing event")
    return handle


def _check_slopes(alibi_slopes: torch.Tensor, H: int) -> None:
    if alibi_slopes.dtype != torch.float32 or tuple(alibi_slopes.shape) != (H,):
        raise ValueError(f"alibi_slopes must be float32 [{H}]")


def decode_dims(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor,
                partition_size: int = 0) -> _lib.DecodeDims:
    S, H, D = q.shape
    d = _lib.DecodeDims()
    d.num_seqs, d.num_heads, d.head_dim = S, H, D
    d.max_blocks_per_seq = block_tables.shape[1]
    d.num_blocks = k_pool.shape[0]
    d.dtype = _DTYPES[q.dtype]
    d.partition_size = partition_size
    return d


def paged_attention_decode_workspace_bytes(q: torch.Tensor, k_pool: torch.Tensor,
                                           block_tables: torch.Tensor,
                                           partition_size: int = 0) -> int:
    d = decode_dims(q, k_pool, block_tables, partition_size)
    n = _lib.load().paged_attention_decode_workspace_bytes(k_pool.shape[2], ctypes.byref(d))
    if n == _lib.SIZE_MAX:
        raise ValueError("invalid shapes for paged_attention_decode")
    return n


def paged_attention_decode_partition_tokens(q: torch.Tensor, k_pool: torch.Tensor,
                                            block_tables: torch.Tensor,
                                            partition_size: int = 0) -> int:
    """Partition size in tokens the library uses for these shapes."""
    d = decode_dims(q, k_pool, block_tables, partition_size)
    n = _lib.load().paged_attention_decode_partition_tokens(k_pool.shape[2], ctypes.byref(d))
    if n < 0:
        raise ValueError("invalid shapes for paged_attention_decode")
    return n


def _decode_call(entry: str, out, q, k_pool, v_pool, block_tables, context_lens, scale,
                 partition_size, workspace, stream, timing_events, alibi_slopes, new_kv=None):
    """Marshal one call of the decode family: paged_attention_decode,
    paged_attention_decode_alibi (with slopes), paged_attention_decode_step
    (with new_kv = (k, v, slot_mapping)) or paged_attention_decode_read_probe,
    which share arguments and checks."""
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("out", out), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if k_pool.shape != v_pool.shape or k_pool.dim() != 4:
        raise ValueError("k_pool and v_pool must both be [num_blocks, num_kv_heads, block_size, head_dim]")
    S, H, D = q.shape
    if out.shape != q.shape or k_pool.shape[3] != D:
        raise ValueError("out must match q, and the pools' head_dim must match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    hkv, bs = k_pool.shape[1], k_pool.shape[2]
    if new_kv is not None:
        k, v, slot_mapping = new_kv
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must have q's dtype")
        if k.shape != (S, hkv, D) or v.shape != (S, hkv, D):
            raise ValueError(f"k and v must be [{S}, {hkv}, {D}] (one new token per sequence)")
        if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
            raise ValueError(f"slot_mapping must be int64 [{S}]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    d = decode_dims(q, k_pool, block_tables, partition_size)
    lib = _lib.load()
    need = lib.paged_attention_decode_workspace_bytes(bs, ctypes.byref(d))
    if need == _lib.SIZE_MAX:
        _check(_lib.PA_ERR_SHAPE, entry)
    if entry == "paged_attention_decode_noalloc":
        # the library's static scratch stands in for the workspace
        if workspace is not None:
            raise ValueError(f"{entry} takes no workspace")
    elif need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        d.workspace = _dev(workspace, "workspace")
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    d.stream = _stream_ptr(stream)
    d.timing_events[0] = _event_ptr(timing_events[0])
    d.timing_events[1] = _event_ptr(timing_events[1])
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
            hkv, ctypes.c_float(scale), bs)
    if new_kv is not None:
        ptrs = ptrs[:2] + (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping")) + \
            ptrs[2:]
    if alibi_slopes is not None:
        _check_slopes(alibi_slopes, H)
        rc = getattr(lib, entry)(*ptrs, _dev(alibi_slopes, "alibi_slopes"), ctypes.byref(d))
    else:
        rc = getattr(lib, entry)(*ptrs, ctypes.byref(d))
    _check(rc, entry)
    return out


def paged_attention_decode(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                           v_pool: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, scale: Optional[float] = None,
                           partition_size: int = 0, workspace: Optional[torch.Tensor] = None,
                           stream=None, timing_events: Sequence = (None, None),
                           alibi_slopes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[S,H,D] <- paged decode attention (see paged_attention_decode in
    include/pagedattn.h).  Pools are [num_blocks, num_kv_heads, block_size,
    head_dim]; the kv-head count and block size are read off k_pool.
    ``scale`` defaults to 1/sqrt(head_dim).  A workspace (unit plan and
    split-K partials) is allocated here when none is given.  With
    ``alibi_slopes`` (fp32 [H]) the call is paged_attention_decode_alibi."""
    entry = "paged_attention_decode" if alibi_slopes is None else "paged_attention_decode_alibi"
    return _decode_call(entry, out, q, k_pool, v_pool, block_tables, context_lens, scale,
                        partition_size, workspace, stream, timing_events, alibi_slopes)


def paged_attention_decode_step(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                                v: torch.Tensor, slot_mapping: torch.Tensor,
                                k_pool: torch.Tensor, v_pool: torch.Tensor,
                                block_tables: torch.Tensor, context_lens: torch.Tensor,
                                scale: Optional[float] = None, partition_size: int = 0,
                                workspace: Optional[torch.Tensor] = None, stream=None,
                                timing_events: Sequence = (None, None)) -> torch.Tensor:
    """One decode step (see paged_attention_decode_step in include/pagedattn.h):
    k[s], v[s] ([S, num_kv_heads, head_dim]) to pool slot slot_mapping[s],
    then out[S,H,D] <- paged decode attention over the updated pools; bit for
    bit reshape_and_cache followed by paged_attention_decode, in one launch
    fewer."""
    return _decode_call("paged_attention_decode_step", out, q, k_pool, v_pool, block_tables,
                        context_lens, scale, partition_size, workspace, stream, timing_events,
                        None, new_kv=(k, v, slot_mapping))


def paged_attention_decode_noalloc(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                                   v_pool: torch.Tensor, block_tables: torch.Tensor,
                                   context_lens: torch.Tensor, scale: Optional[float] = None,
                                   partition_size: int = 0, stream=None,
                                   timing_events: Sequence = (None, None)) -> torch.Tensor:
    """paged_attention_decode with the library's static device scratch in
    place of a workspace (see paged_attention_decode_noalloc in
    include/pagedattn.h): nothing is allocated, here or in the library."""
    return _decode_call("paged_attention_decode_noalloc", out, q, k_pool, v_pool, block_tables,
                        context_lens, scale, partition_size, None, stream, timing_events, None)


def paged_attention_decode_read_probe(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                                      v_pool: torch.Tensor, block_tables: torch.Tensor,
                                      context_lens: torch.Tensor, partition_size: int = 0,
                                      workspace: Optional[torch.Tensor] = None, stream=None,
                                      timing_events: Sequence = (None, None)) -> torch.Tensor:
    """The decode access pattern without its arithmetic (see
    paged_attention_decode_read_probe in include/pagedattn.h): same
    arguments as paged_attention_decode; ``out`` receives one XOR word per
    item, not attention."""
    return _decode_call("paged_attention_decode_read_probe", out, q, k_pool, v_pool,
                        block_tables, context_lens, None, partition_size, workspace, stream,
                        timing_events, None)


def _shared_prefix_call(entry, out, q, k_pool, v_pool, block_tables, context_lens,
                        group_starts, prefix_lens, scale, partition_size, workspace, stream,
                        timing_events, new_kv=None):
    """Marshal paged_attention_decode_shared_prefix, or with new_kv = (k, v,
    slot_mapping) paged_attention_decode_shared_prefix_step."""
    if q.dtype != torch.bfloat16:
        raise ValueError("shared-prefix decode is built for bf16")
    for name, t in (("out", out), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("group_starts", group_starts), ("prefix_lens", prefix_lens)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if group_starts.dim() != 1 or prefix_lens.shape != (group_starts.shape[0] - 1,):
        raise ValueError("group_starts must be [G + 1] and prefix_lens [G]")
    S, H, D = q.shape
    if out.shape != q.shape or k_pool.shape != v_pool.shape or k_pool.dim() != 4 \
            or k_pool.shape[3] != D or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("shapes as for paged_attention_decode")
    hkv, bs = k_pool.shape[1], k_pool.shape[2]
    if new_kv is not None:
        k, v, slot_mapping = new_kv
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must have q's dtype")
        if k.shape != (S, hkv, D) or v.shape != (S, hkv, D):
            raise ValueError(f"k and v must be [{S}, {hkv}, {D}] (one new token per sequence)")
        if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (S,):
            raise ValueError(f"slot_mapping must be int64 [{S}]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    d = decode_dims(q, k_pool, block_tables, partition_size)
    lib = _lib.load()
    need = lib.paged_attention_decode_shared_prefix_workspace_bytes(bs, ctypes.byref(d))
    if need == _lib.SIZE_MAX:
        _check(_lib.PA_ERR_SHAPE, entry)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        d.workspace = _dev(workspace, "workspace")
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    d.stream = _stream_ptr(stream)
    d.timing_events[0] = _event_ptr(timing_events[0])
    d.timing_events[1] = _event_ptr(timing_events[1])
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"), hkv,
            ctypes.c_float(scale), bs, _dev(group_starts, "group_starts"),
            _dev(prefix_lens, "prefix_lens"), prefix_lens.shape[0])
    if new_kv is not None:
        ptrs = ptrs[:2] + (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping")) + \
            ptrs[2:]
    rc = getattr(lib, entry)(*ptrs, ctypes.byref(d))
    _check(rc, entry)
    return out


def paged_attention_decode_shared_prefix(
        out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
        block_tables: torch.Tensor, context_lens: torch.Tensor, group_starts: torch.Tensor,
        prefix_lens: torch.Tensor, scale: Optional[float] = None, partition_size: int = 0,
        workspace: Optional[torch.Tensor] = None, stream=None,
        timing_events: Sequence = (None, None)) -> torch.Tensor:
    """paged_attention_decode for batches whose groups of consecutive
    sequences share prefix pages (see paged_attention_decode_shared_prefix
    in include/pagedattn.h); group_starts int32 [G+1], prefix_lens int32 [G]."""
    return _shared_prefix_call("paged_attention_decode_shared_prefix", out, q, k_pool, v_pool,
                               block_tables, context_lens, group_starts, prefix_lens, scale,
                               partition_size, workspace, stream, timing_events)


def paged_attention_decode_shared_prefix_step(
        out: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
        slot_mapping: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
        block_tables: torch.Tensor, context_lens: torch.Tensor, group_starts: torch.Tensor,
        prefix_lens: torch.Tensor, scale: Optional[float] = None, partition_size: int = 0,
        workspace: Optional[torch.Tensor] = None, stream=None,
        timing_events: Sequence = (None, None)) -> torch.Tensor:
    """One shared-prefix decode step (see
    paged_attention_decode_shared_prefix_step in include/pagedattn.h): the
    new tokens k[s], v[s] to slot_mapping[s], then shared-prefix decode over
    the updated pools; bit for bit reshape_and_cache followed by
    paged_attention_decode_shared_prefix."""
    return _shared_prefix_call("paged_attention_decode_shared_prefix_step", out, q, k_pool,
                               v_pool, block_tables, context_lens, group_starts, prefix_lens,
                               scale, partition_size, workspace, stream, timing_events,
                               new_kv=(k, v, slot_mapping))



def paged_attention_decode_shared_prefix_workspace_bytes(q, k_pool, block_tables,
                                                         partition_size: int = 0) -> int:
    d = decode_dims(q, k_pool, block_tables, partition_size)
    n = _lib.load().paged_attention_decode_shared_prefix_workspace_bytes(k_pool.shape[2],
                                                                         ctypes.byref(d))
    if n == _lib.SIZE_MAX:
        raise ValueError("invalid shapes for paged_attention_decode_shared_prefix")
    return n


def prefill_dims(q: torch.Tensor, k_pool: torch.Tensor, block_tables: torch.Tensor,
                 query_start: torch.Tensor, partition_size: int = 0) -> _lib.PrefillDims:
    T, H, D = q.shape
    d = _lib.PrefillDims()
    d.num_seqs = query_start.shape[0] - 1
    d.num_tokens, d.num_heads, d.head_dim = T, H, D
    d.max_blocks_per_seq = block_tables.shape[1]
    d.num_blocks = k_pool.shape[0]
    d.dtype = _DTYPES[q.dtype]
    d.partition_size = partition_size
    return d


def paged_attention_prefill_workspace_bytes(q: torch.Tensor, k_pool: torch.Tensor,
                                            block_tables: torch.Tensor,
                                            query_start: torch.Tensor,
                                            partition_size: int = 0) -> int:
    d = prefill_dims(q, k_pool, block_tables, query_start, partition_size)
    n = _lib.load().paged_attention_prefill_workspace_bytes(k_pool.shape[1], k_pool.shape[2],
                                                            ctypes.byref(d))
    if n == _lib.SIZE_MAX:
        raise ValueError("invalid shapes for paged_attention_prefill")
    return n


def paged_attention_prefill_partition_tokens(q: torch.Tensor, k_pool: torch.Tensor,
                                             block_tables: torch.Tensor,
                                             query_start: torch.Tensor,
                                             partition_size: int = 0) -> int:
    """Keys per split-K partition that paged_attention_prefill uses for these
    shapes (0: no split)."""
    d = prefill_dims(q, k_pool, block_tables, query_start, partition_size)
    n = _lib.load().paged_attention_prefill_partition_tokens(k_pool.shape[1], k_pool.shape[2],
                                                             ctypes.byref(d))
    if n < 0:
        raise ValueError("invalid shapes for paged_attention_prefill")
    return n


def _prefill_call(entry, out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                  scale, workspace, stream, timing_events, alibi_slopes, partition_size,
                  new_kv=None):
    """Marshal paged_attention_prefill, paged_attention_prefill_alibi (with
    slopes) or, with new_kv = (k, v, slot_mapping),
    paged_attention_prefill_step."""
    if q.dtype != torch.bfloat16:
        raise ValueError("prefill attention is built for bf16")
    for name, t in (("out", out), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    for name, t in (("block_tables", block_tables), ("context_lens", context_lens),
                    ("query_start", query_start)):
        if t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    T, H, D = q.shape
    S = query_start.shape[0] - 1
    if query_start.dim() != 1 or S < 0:
        raise ValueError("query_start must be [S + 1]")
    if out.shape != q.shape or k_pool.shape != v_pool.shape or k_pool.dim() != 4 \
            or k_pool.shape[3] != D:
        raise ValueError("out must match q; pools [num_blocks, num_kv_heads, block_size, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    hkv, bs = k_pool.shape[1], k_pool.shape[2]
    if new_kv is not None:
        k, v, slot_mapping = new_kv
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise ValueError("k and v must have q's dtype")
        if k.shape != (T, hkv, D) or v.shape != (T, hkv, D):
            raise ValueError(f"k and v must be [{T}, {hkv}, {D}] (one row per row of q)")
        if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
            raise ValueError(f"slot_mapping must be int64 [{T}]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    d = prefill_dims(q, k_pool, block_tables, query_start, partition_size)
    lib = _lib.load()
    need = lib.paged_attention_prefill_workspace_bytes(hkv, bs, ctypes.byref(d))
    if need == _lib.SIZE_MAX:
        _check(_lib.PA_ERR_SHAPE, entry)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        d.workspace = _dev(workspace, "workspace")
        d.workspace_bytes = workspace.numel() * workspace.element_size()
    d.stream = _stream_ptr(stream)
    d.timing_events[0] = _event_ptr(timing_events[0])
    d.timing_events[1] = _event_ptr(timing_events[1])
    ptrs = (_dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
            _dev(block_tables, "block_tables"), _dev(context_lens, "context_lens"),
            _dev(query_start, "query_start"), hkv, ctypes.c_float(scale), bs)
    if new_kv is not None:
        ptrs = ptrs[:2] + (_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping")) + \
            ptrs[2:]
    if alibi_slopes is not None:
        _check_slopes(alibi_slopes, H)
        rc = getattr(lib, entry)(*ptrs, _dev(alibi_slopes, "alibi_slopes"), ctypes.byref(d))
    else:
        rc = getattr(lib, entry)(*ptrs, ctypes.byref(d))
    _check(rc, entry)
    return out


def paged_attention_prefill(out: torch.Tensor, q: torch.Tensor, k_pool: torch.Tensor,
                            v_pool: torch.Tensor, block_tables: torch.Tensor,
                            context_lens: torch.Tensor, query_start: torch.Tensor,
                            scale: Optional[float] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None,
                            timing_events: Sequence = (None, None),
                            alibi_slopes: Optional[torch.Tensor] = None,
                            partition_size: int = 0) -> torch.Tensor:
    """out[T,H,D] <- multi-token (prefill / chunked prefill) attention over
    the paged cache (see paged_attention_prefill in include/pagedattn.h);
    query_start int32 [S + 1] gives each sequence's first row of q.
    partition_size: keys per split-K partition (0: the library's choice).  A
    workspace (work plan, split-K partials) is allocated here when none is
    given.  With ``alibi_slopes`` (fp32 [H]) the call is
    paged_attention_prefill_alibi."""
    entry = "paged_attention_prefill" if alibi_slopes is None else "paged_attention_prefill_alibi"
    return _prefill_call(entry, out, q, k_pool, v_pool, block_tables, context_lens, query_start,
                         scale, workspace, stream, timing_events, alibi_slopes, partition_size)


def paged_attention_prefill_step(out: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                                 v: torch.Tensor, slot_mapping: torch.Tensor,
                                 k_pool: torch.Tensor, v_pool: torch.Tensor,
                                 block_tables: torch.Tensor, context_lens: torch.Tensor,
                                 query_start: torch.Tensor, scale: Optional[float] = None,
                                 workspace: Optional[torch.Tensor] = None, stream=None,
                                 timing_events: Sequence = (None, None),
                                 partition_size: int = 0) -> torch.Tensor:
    """One chunked-prefill step (see paged_attention_prefill_step in
    include/pagedattn.h): k[r], v[r] ([T, num_kv_heads, head_dim]) to pool
    slot slot_mapping[r], then out[T,H,D] <- prefill attention over the
    updated pools; bit for bit reshape_and_cache followed by
    paged_attention_prefill, in one launch fewer."""
    return _prefill_call("paged_attention_prefill_step", out, q, k_pool, v_pool, block_tables,
                         context_lens, query_start, scale, workspace, stream, timing_events,
                         None, partition_size, new_kv=(k, v, slot_mapping))


def reshape_and_cache(k: torch.Tensor, v: torch.Tensor, k_pool: torch.Tensor,
                      v_pool: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    """Write k[i], v[i] ([T, num_kv_heads, head_dim]) to pool slot
    slot_mapping[i] (see reshape_and_cache in include/pagedattn.h)."""
    if k.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k.dtype}")
    for name, t in (("v", v), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != k.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from k dtype {k.dtype}")
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    if k.shape != v.shape or k.dim() != 3 or k_pool.shape != v_pool.shape or k_pool.dim() != 4:
        raise ValueError("k, v must be [T, Hkv, D] and pools [NB, Hkv, bs, D]")
    T, hkv, D = k.shape
    if k_pool.shape[1] != hkv or k_pool.shape[3] != D or slot_mapping.shape != (T,):
        raise ValueError("shape mismatch between k/v, pools and slot_mapping")
    d = _lib.CacheDims()
    d.num_tokens, d.num_kv_heads, d.head_dim = T, hkv, D
    d.block_size, d.num_blocks = k_pool.shape[2], k_pool.shape[0]
    d.dtype = _DTYPES[k.dtype]
    d.stream = _stream_ptr(stream)
    rc = _lib.load().reshape_and_cache(_dev(k, "k"), _dev(v, "v"), _dev(k_pool, "k_pool"),
                                       _dev(v_pool, "v_pool"), _dev(slot_mapping, "slot_mapping"),
                                       ctypes.byref(d))
    _check(rc, "reshape_and_cache")


def _pool_ptr(t: torch.Tensor, name: str) -> int:
    """Device tensor, or pinned host tensor (mapped into the device's
    address space); pageable host memory is refused by the library."""
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda and not t.is_pinned():
        raise ValueError(f"{name} must be a device tensor or pinned host memory")
    return t.data_ptr()


def reshape_and_cache_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           k_pool: torch.Tensor, v_pool: torch.Tensor, slot_mapping: torch.Tensor,
                           positions: torch.Tensor, cos_sin: torch.Tensor, rot_dim: int,
                           is_neox: bool = True, stream=None) -> None:
    """Rotate q ([T, H, D]) in place and write rotated k with v to the pool
    slots (see reshape_and_cache_rope in include/pagedattn.h); positions
    int64 [T], cos_sin float32 [max_position, rot_dim] (cosines, then
    sines)."""
    for name, t in (("q", q), ("v", v), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype != k.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from k dtype {k.dtype}")
    if k.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k.dtype}")
    if slot_mapping.dtype != torch.int64 or positions.dtype != torch.int64:
        raise ValueError("slot_mapping and positions must be int64")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != rot_dim:
        raise ValueError("cos_sin must be float32 [max_position, rot_dim]")
    T, hkv, D = k.shape
    if v.shape != k.shape or q.dim() != 3 or q.shape[0] != T or q.shape[2] != D \
            or slot_mapping.shape != (T,) or positions.shape != (T,):
        raise ValueError("q [T, H, D], k and v [T, Hkv, D], slot_mapping and positions [T]")
    d = _lib.CacheDims()
    d.num_tokens, d.num_kv_heads, d.head_dim = T, hkv, D
    d.block_size, d.num_blocks, d.dtype = k_pool.shape[2], k_pool.shape[0], _DTYPES[k.dtype]
    d.stream = _stream_ptr(stream)
    r = _lib.RopeDims()
    r.num_heads, r.rot_dim, r.max_position, r.is_neox = q.shape[1], rot_dim, cos_sin.shape[0], int(is_neox)
    rc = _lib.load().reshape_and_cache_rope(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(slot_mapping, "slot_mapping"), _dev(positions, "positions"), _dev(cos_sin, "cos_sin"),
        ctypes.byref(r), ctypes.byref(d))
    _check(rc, "reshape_and_cache_rope")


def copy_blocks(k_src: torch.Tensor, v_src: torch.Tensor, k_dst: torch.Tensor,
                v_dst: torch.Tensor, block_mapping: torch.Tensor, stream=None) -> None:
    """Copy page block_mapping[i, 0] of the source pools to page
    block_mapping[i, 1] of the destination pools (see copy_blocks in
    include/pagedattn.h).  Pools are [num_blocks, num_kv_heads, block_size,
    head_dim], on the device or in pinned host memory."""
    for name, t in (("v_src", v_src), ("k_dst", k_dst), ("v_dst", v_dst)):
        if t.dtype != k_src.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from k_src dtype {k_src.dtype}")
    if k_src.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_src.dtype}")
    if block_mapping.dtype != torch.int64 or block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be int64 [num_pairs, 2]")
    if k_src.shape != v_src.shape or k_dst.shape != v_dst.shape or k_src.dim() != 4 \
            or k_src.shape[1:] != k_dst.shape[1:]:
        raise ValueError("pools must be [num_blocks, num_kv_heads, block_size, head_dim] "
                         "with matching page shapes")
    d = _lib.CopyDims()
    d.num_pairs = block_mapping.shape[0]
    d.num_kv_heads, d.block_size, d.head_dim = k_src.shape[1], k_src.shape[2], k_src.shape[3]
    d.dtype = _DTYPES[k_src.dtype]
    d.src_num_blocks, d.dst_num_blocks = k_src.shape[0], k_dst.shape[0]
    d.stream = _stream_ptr(stream)
    rc = _lib.load().copy_blocks(_pool_ptr(k_src, "k_src"), _pool_ptr(v_src, "v_src"),
                                 _pool_ptr(k_dst, "k_dst"), _pool_ptr(v_dst, "v_dst"),
                                 _pool_ptr(block_mapping, "block_mapping"), ctypes.byref(d))
    _check(rc, "copy_blocks")


def hbm_read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Stream all of ``buf`` through the read-bandwidth probe kernel."""
    lib = _lib.load()
    if sink is None:
        sink = torch.empty(lib.pa_hbm_read_probe_sink_bytes(), dtype=torch.uint8, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    rc = lib.pa_hbm_read_probe(_dev(buf, "buf"), nbytes - nbytes % 16, _dev(sink, "sink"),
                               _stream_ptr(stream))
    _check(rc, "pa_hbm_read_probe")
    return sink
