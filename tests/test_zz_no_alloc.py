"""paged_attention_decode_noalloc (the library's static device scratch in
place of a caller workspace) against paged_attention_decode with a
workspace, through the C ABI.

The two entry points run the same kernels on the same inputs, so their
outputs must agree bit for bit.  Calls follow each other on one device: the
first is the largest (256 sequences, 4 split-K partitions: 17 MB of
partials), the later ones smaller, so each runs on a scratch that still
holds the previous call's plan and partials.
"""
import ctypes

import numpy as np
import pytest
import torch

from paged_kv_cache_457_amd import _lib, binding
from paged_kv_cache_457_amd.device_inputs import to_host, upload
from paged_kv_cache_457_amd.workloads import build_workload, make_config

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _dims(dw, partition_size, workspace=None):
    w = dw.w
    d = _lib.DecodeDims()
    d.num_seqs, d.num_heads, d.head_dim = w.num_seqs, w.num_heads, w.head_dim
    d.max_blocks_per_seq, d.num_blocks = w.block_tables.shape[1], w.num_blocks
    d.dtype = _lib.PA_DTYPE_BF16 if w.dtype == "bf16" else _lib.PA_DTYPE_F32
    d.partition_size = partition_size
    if workspace is not None:
        d.workspace = workspace.data_ptr()
        d.workspace_bytes = workspace.numel()
    d.stream = torch.cuda.current_stream().cuda_stream
    return d


def _call(entry, dw, d):
    w = dw.w
    lib = _lib.load()
    return getattr(lib, entry)(dw.out.data_ptr(), dw.q.data_ptr(), dw.k_pool.data_ptr(),
                               dw.v_pool.data_ptr(), dw.block_tables.data_ptr(),
                               dw.context_lens.data_ptr(), w.num_kv_heads,
                               ctypes.c_float(float(w.scale)), w.block_size, ctypes.byref(d))


def _both(w, partition_size=0):
    """Output bits of the workspace entry, then of the no-allocation entry
    (the output buffer is poisoned in between)."""
    dw = upload(w)
    binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool, dw.slot_mapping)
    lib = _lib.load()
    d = _dims(dw, partition_size)
    need = lib.paged_attention_decode_workspace_bytes(w.block_size, ctypes.byref(d))
    assert need != _lib.SIZE_MAX and need <= _lib.PA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    rc = _call("paged_attention_decode", dw, _dims(dw, partition_size, ws))
    assert rc == _lib.PA_OK, _lib.status_string(rc)
    torch.cuda.synchronize()
    want = to_host(dw.out, w.dtype).copy()
    dw.out.fill_(float("nan"))
    rc = _call("paged_attention_decode_noalloc", dw, _dims(dw, partition_size))
    assert rc == _lib.PA_OK, _lib.status_string(rc)
    torch.cuda.synchronize()
    got = to_host(dw.out, w.dtype)
    say(f"{w.name}: {w.num_seqs} sequences, workspace {need} bytes")
    return got, want


def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    # 1: 256 lognormal sequences, 32/8 heads, default partitions of 2048
    #    tokens (up to 4 per sequence): the grouped-query kernel and the
    #    split-K merge, 17 MB of partials in the scratch
    w1 = make_config(3)
    got, want = _both(w1)
    assert got.tobytes() == want.tobytes()
    # 2: a smaller call right after, on the scratch the first one filled:
    #    ragged bf16 sequences with one query head per kv-head (the VALU
    #    kernel), 64-token partitions, so fewer, differently placed partials
    w2 = build_workload("noalloc-small", [0, 1, 17, 300, 777, 64, 65], 8, 8, 128, 16, "bf16",
                        seed=11, max_blocks_per_seq=64)
    got, want = _both(w2, partition_size=64)
    assert got.tobytes() == want.tobytes()
    # 3: smaller again: fp32, one partition per sequence (no merge)
    w3 = make_config(1)
    got, want = _both(w3)
    assert got.tobytes() == want.tobytes()
