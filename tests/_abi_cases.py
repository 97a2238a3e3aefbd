"""Host-side argument checks of libpagedattn, run as a child process.

tests/test_abi.py runs this file with every GPU hidden from the HIP runtime,
so even a check that wrongly passed could not reach a device.  Each case
passes stand-in (non-NULL, never dereferenced) pointers and expects a given
status code.  Prints one line per case and exits nonzero on any mismatch.

With a library path as its argument it runs against that build instead: the
host code built with the address and undefined-behaviour sanitizers over
stand-in launches (tests/host_check/pa_stubs.cpp).  There, calls that pass
validation "launch" harmlessly, so further cases check the workspace layout
against the sizes the queries report, and the PA_DEBUG_CHECKS=1 pass on
tables held in host memory.
"""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from paged_kv_cache_457_amd import _lib  # noqa: E402

STUB = len(sys.argv) > 1
lib = _lib.bind(ctypes.CDLL(sys.argv[1])) if STUB else _lib.load()
P = 0x10000          # a 64 KiB-aligned stand-in address; never dereferenced
MIS = P + 4          # misaligned for 16-byte data

failures = 0


def expect(name, got, want):
    global failures
    ok = got == want
    failures += not ok
    print(f"{'ok ' if ok else 'BAD'} {name}: got {got} want {want}", flush=True)


def dims(**kw):
    d = _lib.DecodeDims()
    d.num_seqs, d.num_heads, d.head_dim = 0, 32, 128
    d.max_blocks_per_seq, d.num_blocks, d.dtype = 128, 1000, _lib.PA_DTYPE_BF16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def decode(d, hkv=32, bs=16, scale=0.088, ptrs=None):
    p = ptrs or [P] * 6
    return lib.paged_attention_decode(*p, hkv, ctypes.c_float(scale), bs, ctypes.byref(d))


def cache(**kw):
    d = _lib.CacheDims()
    d.num_tokens, d.num_kv_heads, d.head_dim, d.block_size = 0, 8, 128, 16
    d.num_blocks, d.dtype = 100, _lib.PA_DTYPE_BF16
    ptrs = kw.pop("ptrs", [P] * 5)
    for k, v in kw.items():
        setattr(d, k, v)
    return lib.reshape_and_cache(*ptrs, ctypes.byref(d))


# ---- decode: shape cases use num_seqs == 0, so a check that wrongly passed
# would end in a no-op; pointer cases need num_seqs >= 1 (an empty batch
# accepts NULL pointers) and rely on the hidden GPUs.
ONE = dict(num_seqs=1, max_blocks_per_seq=16)
expect("dims NULL", lib.paged_attention_decode(P, P, P, P, P, P, 32, ctypes.c_float(1), 16, None),
       _lib.PA_ERR_NULL)
for i in range(6):
    ptrs = [P] * 6
    ptrs[i] = None
    expect(f"decode pointer {i} NULL", decode(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
expect("valid empty batch is a no-op", decode(dims()), _lib.PA_OK)
expect("empty batch accepts NULL pointers", decode(dims(), ptrs=[None] * 6), _lib.PA_OK)
expect("negative num_seqs", decode(dims(num_seqs=-1)), _lib.PA_ERR_SHAPE)
expect("zero heads", decode(dims(num_heads=0)), _lib.PA_ERR_SHAPE)
expect("zero kv heads", decode(dims(), hkv=0), _lib.PA_ERR_SHAPE)
expect("H not a multiple of Hkv", decode(dims(num_heads=30), hkv=8), _lib.PA_ERR_SHAPE)
expect("group 3 unsupported", decode(dims(num_heads=24), hkv=8), _lib.PA_ERR_UNSUPPORTED)
expect("group 16 unsupported", decode(dims(num_heads=32), hkv=2), _lib.PA_ERR_UNSUPPORTED)
expect("head_dim 96 unsupported", decode(dims(head_dim=96)), _lib.PA_ERR_UNSUPPORTED)
expect("block_size 8 unsupported", decode(dims(), bs=8), _lib.PA_ERR_UNSUPPORTED)
expect("dtype 7 unsupported", decode(dims(dtype=7)), _lib.PA_ERR_UNSUPPORTED)
expect("zero max_blocks", decode(dims(max_blocks_per_seq=0)), _lib.PA_ERR_SHAPE)
expect("zero num_blocks", decode(dims(num_blocks=0)), _lib.PA_ERR_SHAPE)
expect("reserved nonzero", decode(dims(reserved=1)), _lib.PA_ERR_SHAPE)
expect("partition not a page multiple", decode(dims(partition_size=100)), _lib.PA_ERR_SHAPE)
expect("partition over 256 pages", decode(dims(partition_size=16 * 257)), _lib.PA_ERR_SHAPE)
expect("partition of 256 pages", decode(dims(partition_size=16 * 256)), _lib.PA_OK)
expect("negative partition", decode(dims(partition_size=-16)), _lib.PA_ERR_SHAPE)
expect("scale NaN", decode(dims(), scale=float("nan")), _lib.PA_ERR_SHAPE)
expect("scale inf", decode(dims(), scale=float("inf")), _lib.PA_ERR_SHAPE)
for i in range(4):
    ptrs = [P] * 6
    ptrs[i] = MIS
    expect(f"decode pointer {i} misaligned", decode(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)
ptrs = [P] * 6
ptrs[4] = P + 2
expect("block_tables misaligned", decode(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)

# workspace cases: every call with num_seqs > 0 needs one (the unit plan,
# plus split-K partials when a sequence can span more than one partition);
# each case still fails validation (missing / small / misaligned workspace)
def plan_bytes(S, parts):
    return -(-(4 + S * parts) * 4 // 256) * 256


need_d = dims(num_seqs=4, max_blocks_per_seq=256)
need = lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(need_d))
# 4 sequences of up to 4096 tokens: the default halves 2048 -> 256 tokens
# looking for 128 units and stops at 256: 16 partitions
expect("workspace bytes formula", need,
       plan_bytes(4, 16) + 4 * 32 * 16 * (128 + 2) * 4)
expect("workspace missing", decode(dims(num_seqs=4)), _lib.PA_ERR_WORKSPACE)
expect("workspace missing, one partition", decode(dims(**ONE)), _lib.PA_ERR_WORKSPACE)
expect("workspace too small",
       decode(dims(num_seqs=4, max_blocks_per_seq=256, workspace=P, workspace_bytes=need - 4)),
       _lib.PA_ERR_WORKSPACE)
expect("workspace misaligned",
       decode(dims(num_seqs=4, max_blocks_per_seq=256, workspace=P + 8, workspace_bytes=need + 64)),
       _lib.PA_ERR_WORKSPACE)
expect("one partition: the workspace holds only the plan",
       lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(dims(num_seqs=4, max_blocks_per_seq=16))),
       plan_bytes(4, 1))
expect("empty batch needs no workspace",
       lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(dims(num_seqs=0))), 0)
expect("workspace bytes, partition 512 at bs 32",
       lib.paged_attention_decode_workspace_bytes(32, ctypes.byref(
           dims(num_seqs=8, max_blocks_per_seq=1024, partition_size=512))),
       plan_bytes(8, 64) + 8 * 32 * 64 * 130 * 4)
expect("too many work items",
       decode(dims(num_seqs=1 << 20, max_blocks_per_seq=1 << 14, partition_size=16), hkv=32),
       _lib.PA_ERR_SHAPE)
expect("workspace query rejects bad dims",
       lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(dims(head_dim=80))), _lib.SIZE_MAX)
expect("workspace query rejects NULL", lib.paged_attention_decode_workspace_bytes(16, None), _lib.SIZE_MAX)

# ---- effective partition size
pt = lib.paged_attention_decode_partition_tokens
expect("default partition: table of 2048 tokens is one partition",
       pt(16, ctypes.byref(dims(max_blocks_per_seq=128))), 2048)
expect("default partition: large batch, long runs",
       pt(16, ctypes.byref(dims(num_seqs=256, max_blocks_per_seq=512))), 2048)
expect("default partition: 8 x 32768 tokens at bs 32 keeps 2048",
       pt(32, ctypes.byref(dims(num_seqs=8, max_blocks_per_seq=1024))), 2048)
expect("default partition: 4 x 32768 halves once",
       pt(32, ctypes.byref(dims(num_seqs=4, max_blocks_per_seq=1024))), 1024)
expect("default partition: one long sequence goes to the 256-token floor",
       pt(32, ctypes.byref(dims(num_seqs=1, max_blocks_per_seq=1024))), 256)
expect("default partition: just past one partition, 64 x 2 units",
       pt(16, ctypes.byref(dims(num_seqs=64, max_blocks_per_seq=129))), 2048)
expect("default partition: just past one partition, 16 sequences halve to 256",
       pt(16, ctypes.byref(dims(num_seqs=16, max_blocks_per_seq=129))), 256)
expect("explicit partition", pt(32, ctypes.byref(dims(max_blocks_per_seq=1024, partition_size=512))), 512)
expect("partition query rejects bad dims", pt(16, ctypes.byref(dims(head_dim=80))), -1)
expect("workspace for a one-partition default table",
       lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(dims(num_seqs=4, max_blocks_per_seq=128))),
       plan_bytes(4, 1))

# ---- reshape_and_cache (num_tokens == 0: a wrong pass is a no-op)
expect("cache dims NULL", lib.reshape_and_cache(P, P, P, P, P, None), _lib.PA_ERR_NULL)
for i in range(5):
    ptrs = [P] * 5
    ptrs[i] = None
    expect(f"cache pointer {i} NULL", cache(num_tokens=1, ptrs=ptrs), _lib.PA_ERR_NULL)
expect("valid empty cache write is a no-op", cache(), _lib.PA_OK)
expect("empty cache write accepts NULL pointers", cache(ptrs=[None] * 5), _lib.PA_OK)
expect("negative tokens", cache(num_tokens=-2), _lib.PA_ERR_SHAPE)
expect("zero kv heads", cache(num_kv_heads=0), _lib.PA_ERR_SHAPE)
expect("zero blocks", cache(num_blocks=0), _lib.PA_ERR_SHAPE)
expect("cache head_dim 32", cache(head_dim=32), _lib.PA_ERR_UNSUPPORTED)
expect("cache block_size 64", cache(block_size=64), _lib.PA_ERR_UNSUPPORTED)
expect("cache dtype 5", cache(dtype=5), _lib.PA_ERR_UNSUPPORTED)
for i in range(4):
    ptrs = [P] * 5
    ptrs[i] = MIS
    expect(f"cache pointer {i} misaligned", cache(num_tokens=1, ptrs=ptrs), _lib.PA_ERR_ALIGN)
expect("slot_mapping misaligned", cache(num_tokens=1, ptrs=[P, P, P, P, P + 4]), _lib.PA_ERR_ALIGN)

# ---- shared-prefix decode (valid num_seqs == 0 calls are no-ops)
def shared(d, hkv=32, ptrs=None, groups=1):
    p = ptrs or [P] * 8
    return lib.paged_attention_decode_shared_prefix(*p[:6], hkv, ctypes.c_float(0.088), 16,
                                                    p[6], p[7], groups, ctypes.byref(d))


expect("shared: valid empty batch", shared(dims()), _lib.PA_OK)
expect("shared: empty batch accepts NULL pointers", shared(dims(), ptrs=[None] * 8), _lib.PA_OK)
expect("shared: fp32 unsupported", shared(dims(dtype=_lib.PA_DTYPE_F32, **ONE)), _lib.PA_ERR_UNSUPPORTED)
expect("shared: no groups", shared(dims(**ONE), groups=0), _lib.PA_ERR_SHAPE)
expect("shared: negative groups", shared(dims(), groups=-1), _lib.PA_ERR_SHAPE)
for i in range(8):
    ptrs = [P] * 8
    ptrs[i] = None
    expect(f"shared: pointer {i} NULL", shared(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
for i in (6, 7):
    ptrs = [P] * 8
    ptrs[i] = P + 2
    expect(f"shared: pointer {i} misaligned", shared(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)
expect("shared: workspace missing", shared(dims(**ONE)), _lib.PA_ERR_WORKSPACE)
sp_need = lib.paged_attention_decode_shared_prefix_workspace_bytes(16, ctypes.byref(dims(num_seqs=4)))
# default shared partition 512 tokens: P = 2048 / 512 = 4 -> 8 slots per sequence
expect("shared: workspace bytes formula", sp_need,
       -(-(4 + 5 * 4 * 8 + 2 * 4) * 4 // 256) * 256 + 4 * 32 * 8 * 130 * 4)
expect("shared: workspace too small",
       shared(dims(num_seqs=4, workspace=P, workspace_bytes=sp_need - 4)), _lib.PA_ERR_WORKSPACE)
expect("shared: workspace query rejects bad dims",
       lib.paged_attention_decode_shared_prefix_workspace_bytes(16, ctypes.byref(dims(head_dim=80))),
       _lib.SIZE_MAX)

# ---- copy_blocks (num_pairs == 0: a wrong pass is a no-op)
def copy(ptrs=None, **kw):
    d = _lib.CopyDims()
    d.num_pairs, d.num_kv_heads, d.head_dim, d.block_size = 0, 8, 128, 16
    d.dtype, d.src_num_blocks, d.dst_num_blocks = _lib.PA_DTYPE_BF16, 100, 50
    for k, v in kw.items():
        setattr(d, k, v)
    return lib.copy_blocks(*(ptrs or [P] * 5), ctypes.byref(d))


expect("copy dims NULL", lib.copy_blocks(P, P, P, P, P, None), _lib.PA_ERR_NULL)
expect("valid empty copy is a no-op", copy(), _lib.PA_OK)
expect("empty copy accepts NULL pointers", copy(ptrs=[None] * 5), _lib.PA_OK)
for i in range(5):
    ptrs = [P] * 5
    ptrs[i] = None
    expect(f"copy pointer {i} NULL", copy(ptrs=ptrs, num_pairs=1), _lib.PA_ERR_NULL)
for i in range(4):
    ptrs = [P] * 5
    ptrs[i] = MIS
    expect(f"copy pointer {i} misaligned", copy(ptrs=ptrs, num_pairs=1), _lib.PA_ERR_ALIGN)
expect("copy mapping misaligned", copy(ptrs=[P, P, P, P, P + 4], num_pairs=1), _lib.PA_ERR_ALIGN)
expect("copy negative pairs", copy(num_pairs=-1), _lib.PA_ERR_SHAPE)
expect("copy zero kv heads", copy(num_kv_heads=0), _lib.PA_ERR_SHAPE)
expect("copy zero source blocks", copy(src_num_blocks=0), _lib.PA_ERR_SHAPE)
expect("copy zero destination blocks", copy(dst_num_blocks=0), _lib.PA_ERR_SHAPE)
expect("copy reserved nonzero", copy(reserved=2), _lib.PA_ERR_SHAPE)
expect("copy head_dim 96", copy(head_dim=96), _lib.PA_ERR_UNSUPPORTED)
expect("copy block_size 8", copy(block_size=8), _lib.PA_ERR_UNSUPPORTED)
expect("copy dtype 3", copy(dtype=3), _lib.PA_ERR_UNSUPPORTED)

# ---- prefill (num_tokens == 0 calls are no-ops)
def pdims(**kw):
    d = _lib.PrefillDims()
    d.num_seqs, d.num_tokens, d.num_heads, d.head_dim = 0, 0, 32, 128
    d.max_blocks_per_seq, d.num_blocks, d.dtype = 128, 1000, _lib.PA_DTYPE_BF16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def prefill(d, hkv=8, bs=16, scale=0.088, ptrs=None):
    p = ptrs or [P] * 7
    return lib.paged_attention_prefill(*p, hkv, ctypes.c_float(scale), bs, ctypes.byref(d))


ROWS = dict(num_seqs=2, num_tokens=100)
expect("prefill dims NULL",
       lib.paged_attention_prefill(P, P, P, P, P, P, P, 8, ctypes.c_float(1), 16, None),
       _lib.PA_ERR_NULL)
expect("prefill: valid empty step", prefill(pdims()), _lib.PA_OK)
expect("prefill: empty step accepts NULL pointers", prefill(pdims(), ptrs=[None] * 7), _lib.PA_OK)
expect("prefill: fp32 unsupported", prefill(pdims(dtype=_lib.PA_DTYPE_F32)), _lib.PA_ERR_UNSUPPORTED)
expect("prefill: head_dim 96", prefill(pdims(head_dim=96)), _lib.PA_ERR_UNSUPPORTED)
expect("prefill: block_size 8", prefill(pdims(), bs=8), _lib.PA_ERR_UNSUPPORTED)
expect("prefill: group 3", prefill(pdims(num_heads=6), hkv=2), _lib.PA_ERR_UNSUPPORTED)
expect("prefill: heads not a multiple", prefill(pdims(num_heads=30)), _lib.PA_ERR_SHAPE)
expect("prefill: negative rows", prefill(pdims(num_tokens=-1)), _lib.PA_ERR_SHAPE)
expect("prefill: negative sequences", prefill(pdims(num_seqs=-1)), _lib.PA_ERR_SHAPE)
expect("prefill: rows without sequences", prefill(pdims(num_tokens=5)), _lib.PA_ERR_SHAPE)
expect("prefill: partition not a multiple of the 128-key tile",
       prefill(pdims(partition_size=192)), _lib.PA_ERR_SHAPE)
expect("prefill: negative partition", prefill(pdims(partition_size=-128)), _lib.PA_ERR_SHAPE)
expect("prefill: zero blocks", prefill(pdims(num_blocks=0)), _lib.PA_ERR_SHAPE)
expect("prefill: zero table columns", prefill(pdims(max_blocks_per_seq=0)), _lib.PA_ERR_SHAPE)
expect("prefill: zero kv heads", prefill(pdims(), hkv=0), _lib.PA_ERR_SHAPE)
expect("prefill: NaN scale", prefill(pdims(**ROWS), scale=float("nan")), _lib.PA_ERR_SHAPE)
for i in range(7):
    ptrs = [P] * 7
    ptrs[i] = None
    expect(f"prefill: pointer {i} NULL", prefill(pdims(**ROWS), ptrs=ptrs), _lib.PA_ERR_NULL)
for i in range(7):
    ptrs = [P] * 7
    ptrs[i] = MIS + 2 if i >= 4 else MIS
    expect(f"prefill: pointer {i} misaligned", prefill(pdims(**ROWS), ptrs=ptrs), _lib.PA_ERR_ALIGN)
expect("prefill: workspace missing", prefill(pdims(**ROWS)), _lib.PA_ERR_WORKSPACE)
# plan ints 4 + 8 * rows * P + rows (rounded to 256 bytes), plus with P > 1
# partitions the partials rows * heads * P * (head_dim + 2) floats
def pf_bytes(rows, heads, dh, parts):
    b = -(-(4 + 8 * rows * parts + rows) * 4 // 256) * 256
    return b + (rows * heads * parts * (dh + 2) * 4 if parts > 1 else 0)


pf_short = lib.paged_attention_prefill_workspace_bytes(
    8, 16, ctypes.byref(pdims(max_blocks_per_seq=64, **ROWS)))
expect("prefill: workspace bytes, capacity 1024 keys is never split", pf_short,
       pf_bytes(100, 32, 128, 1))
pf_need = lib.paged_attention_prefill_workspace_bytes(8, 16, ctypes.byref(pdims(**ROWS)))
# 100 rows, group 4: 2 blocks x 8 kv heads = 16 items; capacity 2048 keys,
# partitions of max(1024, 2048 / 64) = 1024 keys -> P = 2
expect("prefill: workspace bytes, default split", pf_need, pf_bytes(100, 32, 128, 2))
expect("prefill: workspace bytes, explicit partition 384",
       lib.paged_attention_prefill_workspace_bytes(
           8, 16, ctypes.byref(pdims(partition_size=384, **ROWS))), pf_bytes(100, 32, 128, 6))
expect("prefill: too many items for int32",
       lib.paged_attention_prefill_workspace_bytes(
           8, 16, ctypes.byref(pdims(num_seqs=1, num_tokens=1 << 24, max_blocks_per_seq=1 << 12,
                                     partition_size=128))), _lib.SIZE_MAX)
ppt = lib.paged_attention_prefill_partition_tokens
expect("prefill partition: default, few items", ppt(8, 16, ctypes.byref(pdims(**ROWS))), 1024)
expect("prefill partition: default, capacity 1024", ppt(
    8, 16, ctypes.byref(pdims(max_blocks_per_seq=64, **ROWS))), 0)
expect("prefill partition: default, long table", ppt(
    8, 16, ctypes.byref(pdims(num_seqs=1, num_tokens=512, max_blocks_per_seq=2048))), 2048)
expect("prefill partition: default, 1024 items", ppt(
    8, 16, ctypes.byref(pdims(num_seqs=2, num_tokens=8192, max_blocks_per_seq=2048))), 0)
expect("prefill partition: explicit", ppt(8, 16, ctypes.byref(pdims(partition_size=128, **ROWS))),
       128)
expect("prefill partition: explicit beyond the capacity",
       ppt(8, 16, ctypes.byref(pdims(partition_size=4096, **ROWS))), 0)
expect("prefill partition: bad dims", ppt(8, 16, ctypes.byref(pdims(head_dim=80))), -1)
expect("prefill: workspace too small",
       prefill(pdims(workspace=P, workspace_bytes=pf_need - 4, **ROWS)), _lib.PA_ERR_WORKSPACE)
expect("prefill: workspace misaligned",
       prefill(pdims(workspace=MIS, workspace_bytes=pf_need, **ROWS)), _lib.PA_ERR_WORKSPACE)
expect("prefill: workspace query, empty step",
       lib.paged_attention_prefill_workspace_bytes(8, 16, ctypes.byref(pdims())), 0)
expect("prefill: workspace query rejects bad dims",
       lib.paged_attention_prefill_workspace_bytes(8, 16, ctypes.byref(pdims(head_dim=80))),
       _lib.SIZE_MAX)

# ---- ALiBi entry points
def decode_alibi(d, slopes=P, ptrs=None):
    p = ptrs or [P] * 6
    return lib.paged_attention_decode_alibi(*p, 32, ctypes.c_float(0.088), 16, slopes,
                                            ctypes.byref(d))


expect("decode alibi: empty batch, no slopes", decode_alibi(dims(), slopes=None), _lib.PA_OK)
expect("decode alibi: slopes NULL", decode_alibi(dims(**ONE), slopes=None), _lib.PA_ERR_NULL)
expect("decode alibi: slopes misaligned", decode_alibi(dims(**ONE), slopes=P + 2), _lib.PA_ERR_ALIGN)
expect("decode alibi: bad dims first", decode_alibi(dims(head_dim=96, **ONE), slopes=None),
       _lib.PA_ERR_UNSUPPORTED)
expect("decode alibi: workspace missing", decode_alibi(dims(**ONE)), _lib.PA_ERR_WORKSPACE)
expect("decode alibi: dims NULL",
       lib.paged_attention_decode_alibi(P, P, P, P, P, P, 32, ctypes.c_float(1), 16, P, None),
       _lib.PA_ERR_NULL)


def prefill_alibi(d, slopes=P):
    return lib.paged_attention_prefill_alibi(*([P] * 7), 8, ctypes.c_float(0.088), 16, slopes,
                                             ctypes.byref(d))


expect("prefill alibi: empty step, no slopes", prefill_alibi(pdims(), slopes=None), _lib.PA_OK)
expect("prefill alibi: slopes NULL", prefill_alibi(pdims(**ROWS), slopes=None), _lib.PA_ERR_NULL)
expect("prefill alibi: slopes misaligned", prefill_alibi(pdims(**ROWS), slopes=P + 1),
       _lib.PA_ERR_ALIGN)
expect("prefill alibi: fp32 unsupported", prefill_alibi(pdims(dtype=_lib.PA_DTYPE_F32, **ROWS)),
       _lib.PA_ERR_UNSUPPORTED)
expect("prefill alibi: workspace missing", prefill_alibi(pdims(**ROWS)), _lib.PA_ERR_WORKSPACE)


# ---- cache write with RoPE (num_tokens == 0: a wrong pass is a no-op)
def rope_call(ptrs=None, r=None, **kw):
    d = _lib.CacheDims()
    d.num_tokens, d.num_kv_heads, d.head_dim, d.block_size = 0, 8, 128, 16
    d.num_blocks, d.dtype = 100, _lib.PA_DTYPE_BF16
    for k, v in kw.items():
        setattr(d, k, v)
    if r is None:
        r = _lib.RopeDims()
        r.num_heads, r.rot_dim, r.max_position, r.is_neox = 32, 128, 4096, 1
    return lib.reshape_and_cache_rope(*(ptrs or [P] * 8), ctypes.byref(r), ctypes.byref(d))


def rdims(**kw):
    r = _lib.RopeDims()
    r.num_heads, r.rot_dim, r.max_position, r.is_neox = 32, 128, 4096, 1
    for k, v in kw.items():
        setattr(r, k, v)
    return r


expect("rope: valid empty write", rope_call(), _lib.PA_OK)
expect("rope: empty write accepts NULL pointers", rope_call(ptrs=[None] * 8), _lib.PA_OK)
expect("rope: rope dims NULL",
       lib.reshape_and_cache_rope(*([P] * 8), None, ctypes.byref(_lib.CacheDims())), _lib.PA_ERR_NULL)
expect("rope: odd rot_dim", rope_call(r=rdims(rot_dim=63)), _lib.PA_ERR_SHAPE)
expect("rope: rot_dim past head_dim", rope_call(r=rdims(rot_dim=256)), _lib.PA_ERR_SHAPE)
expect("rope: rot_dim 24 (not whole chunks)", rope_call(r=rdims(rot_dim=24)), _lib.PA_ERR_UNSUPPORTED)
expect("rope: rot_dim 8 fp32 is whole chunks",
       rope_call(r=rdims(rot_dim=8), dtype=_lib.PA_DTYPE_F32), _lib.PA_OK)
expect("rope: is_neox 2", rope_call(r=rdims(is_neox=2)), _lib.PA_ERR_SHAPE)
expect("rope: reserved", rope_call(r=rdims(reserved=3)), _lib.PA_ERR_SHAPE)
expect("rope: zero positions", rope_call(r=rdims(max_position=0)), _lib.PA_ERR_SHAPE)
expect("rope: zero query heads", rope_call(r=rdims(num_heads=0)), _lib.PA_ERR_SHAPE)
expect("rope: head_dim 96", rope_call(head_dim=96), _lib.PA_ERR_UNSUPPORTED)
for i in range(8):
    ptrs = [P] * 8
    ptrs[i] = None
    expect(f"rope: pointer {i} NULL", rope_call(ptrs=ptrs, num_tokens=1), _lib.PA_ERR_NULL)
for i, bad in ((0, MIS), (1, MIS), (2, MIS), (3, MIS), (4, MIS), (5, P + 4), (6, P + 4), (7, P + 8)):
    ptrs = [P] * 8
    ptrs[i] = bad
    expect(f"rope: pointer {i} misaligned", rope_call(ptrs=ptrs, num_tokens=1), _lib.PA_ERR_ALIGN)

# ---- decode access-pattern probe: the decode call's checks
def read_probe(d, hkv=32, bs=16, ptrs=None):
    p = ptrs or [P] * 6
    return lib.paged_attention_decode_read_probe(*p, hkv, ctypes.c_float(0.088), bs,
                                                 ctypes.byref(d))


expect("read probe dims NULL",
       lib.paged_attention_decode_read_probe(P, P, P, P, P, P, 32, ctypes.c_float(1), 16, None),
       _lib.PA_ERR_NULL)
for i in range(6):
    ptrs = [P] * 6
    ptrs[i] = None
    expect(f"read probe pointer {i} NULL", read_probe(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
expect("read probe empty batch is a no-op", read_probe(dims()), _lib.PA_OK)
expect("read probe group 3 unsupported", read_probe(dims(num_heads=24), hkv=8),
       _lib.PA_ERR_UNSUPPORTED)
expect("read probe block_size 8 unsupported", read_probe(dims(), bs=8), _lib.PA_ERR_UNSUPPORTED)
expect("read probe misaligned k_pool", read_probe(dims(**ONE), ptrs=[P, P, MIS, P, P, P]),
       _lib.PA_ERR_ALIGN)
expect("read probe without workspace", read_probe(dims(**ONE)), _lib.PA_ERR_WORKSPACE)

# ---- decode without a workspace (the library's static scratch); every
# case is rejected before the scratch is looked up, or is an empty batch
def noalloc(d, hkv=32, bs=16, ptrs=None):
    p = ptrs or [P] * 6
    return lib.paged_attention_decode_noalloc(*p, hkv, ctypes.c_float(0.088), bs, ctypes.byref(d))


expect("noalloc dims NULL",
       lib.paged_attention_decode_noalloc(P, P, P, P, P, P, 32, ctypes.c_float(1), 16, None),
       _lib.PA_ERR_NULL)
expect("noalloc empty batch is a no-op", noalloc(dims()), _lib.PA_OK)
expect("noalloc empty batch accepts NULL pointers", noalloc(dims(), ptrs=[None] * 6), _lib.PA_OK)
expect("noalloc rejects a workspace",
       noalloc(dims(**ONE, workspace=P, workspace_bytes=1 << 20)), _lib.PA_ERR_WORKSPACE)
expect("noalloc rejects workspace bytes without a pointer",
       noalloc(dims(**ONE, workspace_bytes=256)), _lib.PA_ERR_WORKSPACE)
for i in range(6):
    ptrs = [P] * 6
    ptrs[i] = None
    expect(f"noalloc pointer {i} NULL", noalloc(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
expect("noalloc misaligned q", noalloc(dims(**ONE), ptrs=[P, MIS, P, P, P, P]), _lib.PA_ERR_ALIGN)
expect("noalloc head_dim 96 unsupported", noalloc(dims(**ONE, head_dim=96)), _lib.PA_ERR_UNSUPPORTED)
# 8192 sequences x 4 heads of 64 dims in 64 one-page partitions: 70 MB of
# partials, over the 32 MiB scratch
big = dims(num_seqs=8192, num_heads=4, head_dim=64, max_blocks_per_seq=64, partition_size=16)
big_need = lib.paged_attention_decode_workspace_bytes(16, ctypes.byref(big))
expect("oversized call needs more than the scratch",
       big_need > _lib.PA_NOALLOC_SCRATCH_BYTES, True)
expect("noalloc oversized call", noalloc(big, hkv=4), _lib.PA_ERR_SCRATCH_LIMIT)
# the largest batch of that shape that fits is not rejected for size: with
# num_blocks = 0 it stops at the shape check instead, which runs first
fit = dims(num_seqs=3000, num_heads=4, head_dim=64, max_blocks_per_seq=64, partition_size=16,
           num_blocks=0)
expect("noalloc shape errors come before the size limit", noalloc(fit, hkv=4), _lib.PA_ERR_SHAPE)

# ---- decode step (cache write, then decode): pointers out, q, k, v,
# slot_mapping, k_pool, v_pool, block_tables, context_lens
def step(d, hkv=32, bs=16, scale=0.088, ptrs=None):
    p = ptrs or [P] * 9
    return lib.paged_attention_decode_step(*p, hkv, ctypes.c_float(scale), bs, ctypes.byref(d))


expect("step dims NULL",
       lib.paged_attention_decode_step(*([P] * 9), 32, ctypes.c_float(1), 16, None),
       _lib.PA_ERR_NULL)
expect("step empty batch is a no-op", step(dims()), _lib.PA_OK)
expect("step empty batch accepts NULL pointers", step(dims(), ptrs=[None] * 9), _lib.PA_OK)
for i in range(9):
    ptrs = [P] * 9
    ptrs[i] = None
    expect(f"step pointer {i} NULL", step(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
for i in (0, 1, 2, 3, 5, 6):
    ptrs = [P] * 9
    ptrs[i] = MIS
    expect(f"step pointer {i} misaligned", step(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)
ptrs = [P] * 9
ptrs[4] = P + 4
expect("step slot_mapping misaligned", step(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)
expect("step head_dim 96 unsupported", step(dims(**ONE, head_dim=96)), _lib.PA_ERR_UNSUPPORTED)
expect("step block_size 8 unsupported", step(dims(**ONE), bs=8), _lib.PA_ERR_UNSUPPORTED)
expect("step group 3 unsupported", step(dims(**ONE, num_heads=24), hkv=8),
       _lib.PA_ERR_UNSUPPORTED)
expect("step scale NaN", step(dims(**ONE), scale=float("nan")), _lib.PA_ERR_SHAPE)
expect("step without workspace", step(dims(**ONE)), _lib.PA_ERR_WORKSPACE)

# ---- shared-prefix step: pointers out, q, k, v, slot_mapping, k_pool,
# v_pool, block_tables, context_lens, then group_starts, prefix_lens
def shared_step(d, ptrs=None, groups=1):
    p = ptrs or [P] * 11
    return lib.paged_attention_decode_shared_prefix_step(
        *p[:9], 32, ctypes.c_float(0.088), 16, p[9], p[10], groups, ctypes.byref(d))


expect("shared step dims NULL", lib.paged_attention_decode_shared_prefix_step(
    *([P] * 9), 32, ctypes.c_float(1), 16, P, P, 1, None), _lib.PA_ERR_NULL)
expect("shared step empty batch accepts NULL pointers", shared_step(dims(), ptrs=[None] * 11),
       _lib.PA_OK)
for i in range(11):
    ptrs = [P] * 11
    ptrs[i] = None
    expect(f"shared step pointer {i} NULL", shared_step(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_NULL)
ptrs = [P] * 11
ptrs[4] = P + 4
expect("shared step slot_mapping misaligned", shared_step(dims(**ONE), ptrs=ptrs), _lib.PA_ERR_ALIGN)
expect("shared step fp32 unsupported", shared_step(dims(**ONE, dtype=_lib.PA_DTYPE_F32)),
       _lib.PA_ERR_UNSUPPORTED)
expect("shared step without workspace", shared_step(dims(**ONE)), _lib.PA_ERR_WORKSPACE)

# ---- prefill step: pointers out, q, k, v, slot_mapping, k_pool, v_pool,
# block_tables, context_lens, query_start
def prefill_step(d, hkv=8, scale=0.088, ptrs=None):
    p = ptrs or [P] * 10
    return lib.paged_attention_prefill_step(*p, hkv, ctypes.c_float(scale), 16, ctypes.byref(d))


expect("prefill step dims NULL", lib.paged_attention_prefill_step(
    *([P] * 10), 8, ctypes.c_float(1), 16, None), _lib.PA_ERR_NULL)
expect("prefill step empty step accepts NULL pointers",
       prefill_step(pdims(), ptrs=[None] * 10), _lib.PA_OK)
for i in range(10):
    ptrs = [P] * 10
    ptrs[i] = None
    expect(f"prefill step pointer {i} NULL", prefill_step(pdims(**ROWS), ptrs=ptrs),
           _lib.PA_ERR_NULL)
for i in (2, 3):
    ptrs = [P] * 10
    ptrs[i] = MIS
    expect(f"prefill step pointer {i} misaligned", prefill_step(pdims(**ROWS), ptrs=ptrs),
           _lib.PA_ERR_ALIGN)
ptrs = [P] * 10
ptrs[4] = P + 4
expect("prefill step slot_mapping misaligned", prefill_step(pdims(**ROWS), ptrs=ptrs),
       _lib.PA_ERR_ALIGN)
expect("prefill step fp32 unsupported", prefill_step(pdims(dtype=_lib.PA_DTYPE_F32, **ROWS)),
       _lib.PA_ERR_UNSUPPORTED)
expect("prefill step NaN scale", prefill_step(pdims(**ROWS), scale=float("nan")),
       _lib.PA_ERR_SHAPE)
expect("prefill step without workspace", prefill_step(pdims(**ROWS)), _lib.PA_ERR_WORKSPACE)

# ---- probe
expect("probe NULL buffer", lib.pa_hbm_read_probe(None, 1024, P, None), _lib.PA_ERR_NULL)
expect("probe size not a multiple of 16", lib.pa_hbm_read_probe(P, 1000, P, None), _lib.PA_ERR_SHAPE)
expect("probe misaligned", lib.pa_hbm_read_probe(MIS, 1024, P, None), _lib.PA_ERR_ALIGN)

# ---- status strings
for rc in range(9):
    s = lib.pa_status_string(rc).decode()
    expect(f"status string {rc}", s.split(":")[0].startswith("PA_"), True)
expect("unknown status", lib.pa_status_string(99).decode(), "unknown status")

if STUB:
    import _abi_stub_cases
    _abi_stub_cases.run(lib, expect)

print(f"{failures} failures", flush=True)
sys.exit(1 if failures else 0)
