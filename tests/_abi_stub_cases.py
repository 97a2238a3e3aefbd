"""Cases that need the host-check build (tests/_abi_cases.py with a library
path): the C ABI's host code over stand-in launches that touch no memory.

* Workspace layout: for calls that pass validation with a workspace of
  exactly the reported size, the plan and partials the launch was given
  must lie inside that workspace (at shapes up to the int32 item limit).
* PA_DEBUG_CHECKS=1: with the tables in host memory (the stand-in copy is a
  memcpy), each violated precondition returns PA_ERR_PRECONDITION and
  launches nothing; valid tables launch once.
"""
import ctypes
import os

from paged_kv_cache_457_amd import _lib

P = 1 << 36                    # stand-in device address, 4 KiB aligned, never dereferenced


def _dims(**kw):
    d = _lib.DecodeDims()
    d.num_seqs, d.num_heads, d.head_dim = 1, 32, 128
    d.max_blocks_per_seq, d.num_blocks, d.dtype = 128, 1000, _lib.PA_DTYPE_BF16
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _span(lib):
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    lib.pa_stub_last_span(ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def _arr(ctype, values):
    a = (ctype * max(1, len(values)))(*values)
    return a, ctypes.addressof(a)


def run(lib, expect):
    lib.pa_stub_launches.restype = ctypes.c_int
    lib.pa_stub_last_span.restype = None
    lib.pa_stub_last_span.argtypes = [ctypes.POINTER(ctypes.c_size_t)] * 2
    launches = lib.pa_stub_launches

    # ---- decode: the launch's plan and partials inside the workspace
    shapes = [
        dict(num_seqs=64, max_blocks_per_seq=128, bs=16, hkv=32),                  # Llama-2-7B
        dict(num_seqs=256, max_blocks_per_seq=512, bs=16, hkv=8),                  # ragged GQA
        dict(num_seqs=8, max_blocks_per_seq=1024, bs=32, hkv=8, partition_size=512),
        dict(num_seqs=3, max_blocks_per_seq=5000, bs=16, hkv=4, num_heads=32, partition_size=16),
        # near the int32 limit of (sequence, partition, kv-head) items
        dict(num_seqs=65536, max_blocks_per_seq=1024, bs=32, hkv=8, partition_size=32),
    ]
    for sh in shapes:
        sh = dict(sh)
        bs, hkv = sh.pop("bs"), sh.pop("hkv")
        d = _dims(**sh)
        need = lib.paged_attention_decode_workspace_bytes(bs, ctypes.byref(d))
        d.workspace, d.workspace_bytes = P, need
        n0 = launches()
        rc = lib.paged_attention_decode(P, P, P, P, P, P, hkv, ctypes.c_float(0.1), bs,
                                        ctypes.byref(d))
        lo, hi = _span(lib)
        expect(f"decode {sh}: launched", (rc, launches() - n0), (_lib.PA_OK, 1))
        expect(f"decode {sh}: plan and partials inside {need} B", P <= lo and hi <= P + need,
               True)
        d.workspace_bytes = need - 1
        expect(f"decode {sh}: one byte short", lib.paged_attention_decode(
            P, P, P, P, P, P, hkv, ctypes.c_float(0.1), bs, ctypes.byref(d)),
            _lib.PA_ERR_WORKSPACE)

    # ---- the static scratch: spans stay inside its 32 MiB
    d = _dims(num_seqs=256, max_blocks_per_seq=512)
    rc = lib.paged_attention_decode_noalloc(P, P, P, P, P, P, 8, ctypes.c_float(0.1), 16,
                                            ctypes.byref(d))
    lo, hi = _span(lib)
    expect("noalloc c3 shape launched", rc, _lib.PA_OK)
    expect("noalloc spans inside the scratch", hi - lo <= _lib.PA_NOALLOC_SCRATCH_BYTES, True)

    # ---- shared prefix
    for sh in (dict(num_seqs=128, max_blocks_per_seq=81), dict(num_seqs=6, max_blocks_per_seq=203,
                                                                partition_size=4096)):
        d = _dims(**sh)
        need = lib.paged_attention_decode_shared_prefix_workspace_bytes(16, ctypes.byref(d))
        d.workspace, d.workspace_bytes = P, need
        rc = lib.paged_attention_decode_shared_prefix(P, P, P, P, P, P, 8, ctypes.c_float(0.1),
                                                      16, P, P, 1, ctypes.byref(d))
        lo, hi = _span(lib)
        expect(f"shared prefix {sh}: launched", rc, _lib.PA_OK)
        expect(f"shared prefix {sh}: inside {need} B", P <= lo and hi <= P + need, True)

    # ---- prefill, unsplit and split
    for sh in (dict(num_seqs=8, num_tokens=8192, max_blocks_per_seq=256),
               dict(num_seqs=2, num_tokens=768, max_blocks_per_seq=1024)):
        d = _lib.PrefillDims()
        d.num_heads, d.head_dim, d.num_blocks, d.dtype = 32, 128, 5000, _lib.PA_DTYPE_BF16
        for k, v in sh.items():
            setattr(d, k, v)
        need = lib.paged_attention_prefill_workspace_bytes(8, 16, ctypes.byref(d))
        d.workspace, d.workspace_bytes = P, need
        rc = lib.paged_attention_prefill(P, P, P, P, P, P, P, 8, ctypes.c_float(0.1), 16,
                                         ctypes.byref(d))
        lo, hi = _span(lib)
        expect(f"prefill {sh}: launched", rc, _lib.PA_OK)
        expect(f"prefill {sh}: inside {need} B", P <= lo and hi <= P + need, True)
        rc = lib.paged_attention_prefill_step(P, P, P, P, P, P, P, P, P, P, 8,
                                              ctypes.c_float(0.1), 16, ctypes.byref(d))
        lo, hi = _span(lib)
        expect(f"prefill step {sh}: launched", rc, _lib.PA_OK)
        expect(f"prefill step {sh}: inside {need} B", P <= lo and hi <= P + need, True)

    # ---- PA_DEBUG_CHECKS=1 on host-resident tables
    bs, mb, nb = 16, 4, 10
    tables = [3, 1, 7, -1,     # ctx 40: 3 pages used, column 3 unused
              2, 9, 0, 5]      # ctx 64: all 4 used
    ctx = [40, 64]

    def decode_with(tab, lens, debug=True):
        if debug:
            os.environ["PA_DEBUG_CHECKS"] = "1"
        else:
            os.environ.pop("PA_DEBUG_CHECKS", None)
        bt, bt_p = _arr(ctypes.c_int32, tab)
        cl, cl_p = _arr(ctypes.c_int32, lens)
        d = _dims(num_seqs=2, num_heads=4, max_blocks_per_seq=mb, num_blocks=nb, workspace=P,
                  workspace_bytes=1 << 20)
        n0 = launches()
        rc = lib.paged_attention_decode(P, P, P, P, bt_p, cl_p, 4, ctypes.c_float(0.1), bs,
                                        ctypes.byref(d))
        return rc, launches() - n0

    expect("debug: valid tables launch", decode_with(tables, ctx), (_lib.PA_OK, 1))
    bad = list(tables)
    bad[1] = nb
    expect("debug: page id past the pool", decode_with(bad, ctx), (_lib.PA_ERR_PRECONDITION, 0))
    bad = list(tables)
    bad[5] = -2
    expect("debug: negative page id", decode_with(bad, ctx), (_lib.PA_ERR_PRECONDITION, 0))
    bad = list(tables)
    bad[3] = 12345
    expect("debug: unused column may hold anything", decode_with(bad, ctx), (_lib.PA_OK, 1))
    expect("debug: context past the table", decode_with(tables, [40, mb * bs + 1]),
           (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: negative context", decode_with(tables, [-1, 64]),
           (_lib.PA_ERR_PRECONDITION, 0))
    bad = list(tables)
    bad[1] = nb
    expect("without PA_DEBUG_CHECKS the kernel's skip applies",
           decode_with(bad, ctx, debug=False), (_lib.PA_OK, 1))
    os.environ["PA_DEBUG_CHECKS"] = "1"

    # cache write slots
    def cache_with(slots):
        sl, sl_p = _arr(ctypes.c_int64, slots)
        d = _lib.CacheDims()
        d.num_tokens, d.num_kv_heads, d.head_dim, d.block_size = len(slots), 8, 128, 16
        d.num_blocks, d.dtype = nb, _lib.PA_DTYPE_BF16
        n0 = launches()
        rc = lib.reshape_and_cache(P, P, P, P, sl_p, ctypes.byref(d))
        return rc, launches() - n0

    expect("debug: distinct slots", cache_with([0, 17, -1, nb * 16 - 1, -1]), (_lib.PA_OK, 1))
    expect("debug: duplicate slot", cache_with([5, 17, 5]), (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: slot past the pool", cache_with([5, nb * 16]), (_lib.PA_ERR_PRECONDITION, 0))

    # decode step: the table and slot checks of both calls, before one launch
    def step_with(tab, lens, slots):
        bt, bt_p = _arr(ctypes.c_int32, tab)
        cl, cl_p = _arr(ctypes.c_int32, lens)
        sl, sl_p = _arr(ctypes.c_int64, slots)
        d = _dims(num_seqs=2, num_heads=4, max_blocks_per_seq=mb, num_blocks=nb, workspace=P,
                  workspace_bytes=1 << 20)
        n0 = launches()
        rc = lib.paged_attention_decode_step(P, P, P, P, sl_p, P, P, bt_p, cl_p, 4,
                                             ctypes.c_float(0.1), bs, ctypes.byref(d))
        return rc, launches() - n0

    expect("debug step: valid tables and slots launch once", step_with(tables, ctx, [3, 40]),
           (_lib.PA_OK, 1))
    expect("debug step: duplicate slot", step_with(tables, ctx, [3, 3]),
           (_lib.PA_ERR_PRECONDITION, 0))
    bad = list(tables)
    bad[1] = nb
    expect("debug step: page id past the pool", step_with(bad, ctx, [3, 40]),
           (_lib.PA_ERR_PRECONDITION, 0))

    # sharing groups
    def shared_with(tab, starts, prefixes, lens):
        bt, bt_p = _arr(ctypes.c_int32, tab)
        cl, cl_p = _arr(ctypes.c_int32, lens)
        gs, gs_p = _arr(ctypes.c_int32, starts)
        pl, pl_p = _arr(ctypes.c_int32, prefixes)
        d = _dims(num_seqs=len(lens), num_heads=8, max_blocks_per_seq=mb, num_blocks=nb,
                  workspace=P, workspace_bytes=1 << 20)
        n0 = launches()
        rc = lib.paged_attention_decode_shared_prefix(P, P, P, P, bt_p, cl_p, 4,
                                                      ctypes.c_float(0.1), bs, gs_p, pl_p,
                                                      len(prefixes), ctypes.byref(d))
        return rc, launches() - n0

    shared = [4, 6, 1, -1,
              4, 6, 8, -1,
              2, 3, -1, -1]     # sequences 0, 1 share 2 pages; 2 alone
    lens = [40, 33, 20]
    expect("debug: valid groups", shared_with(shared, [0, 2, 3], [32, 0], lens), (_lib.PA_OK, 1))
    bad = list(shared)
    bad[5] = 7
    expect("debug: members disagree on a prefix page",
           shared_with(bad, [0, 2, 3], [32, 0], lens), (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: partial prefix page is the members' own",
           shared_with(shared, [0, 2, 3], [40, 0], lens), (_lib.PA_OK, 1))
    expect("debug: groups not ending at num_seqs",
           shared_with(shared, [0, 2, 2], [32, 0], lens), (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: decreasing group starts",
           shared_with(shared, [0, 3, 2], [32, 0], lens), (_lib.PA_ERR_PRECONDITION, 0))

    # prefill query_start
    def prefill_with(qs):
        bt, bt_p = _arr(ctypes.c_int32, tables)
        cl, cl_p = _arr(ctypes.c_int32, ctx)
        q, q_p = _arr(ctypes.c_int32, qs)
        d = _lib.PrefillDims()
        d.num_seqs, d.num_tokens, d.num_heads, d.head_dim = 2, 12, 8, 128
        d.max_blocks_per_seq, d.num_blocks, d.dtype = mb, nb, _lib.PA_DTYPE_BF16
        d.workspace, d.workspace_bytes = P, 1 << 20
        n0 = launches()
        rc = lib.paged_attention_prefill(P, P, P, P, bt_p, cl_p, q_p, 4, ctypes.c_float(0.1),
                                         bs, ctypes.byref(d))
        return rc, launches() - n0

    expect("debug: valid query_start", prefill_with([0, 5, 12]), (_lib.PA_OK, 1))
    expect("debug: decreasing query_start", prefill_with([0, 13, 12]),
           (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: query_start not ending at num_tokens", prefill_with([0, 5, 11]),
           (_lib.PA_ERR_PRECONDITION, 0))

    # prefill step: the query_start, table and slot checks of both calls
    def prefill_step_with(qs, slots):
        bt, bt_p = _arr(ctypes.c_int32, tables)
        cl, cl_p = _arr(ctypes.c_int32, ctx)
        q, q_p = _arr(ctypes.c_int32, qs)
        sl, sl_p = _arr(ctypes.c_int64, slots)
        d = _lib.PrefillDims()
        d.num_seqs, d.num_tokens, d.num_heads, d.head_dim = 2, len(slots), 8, 128
        d.max_blocks_per_seq, d.num_blocks, d.dtype = mb, nb, _lib.PA_DTYPE_BF16
        d.workspace, d.workspace_bytes = P, 1 << 20
        n0 = launches()
        rc = lib.paged_attention_prefill_step(P, P, P, P, sl_p, P, P, bt_p, cl_p, q_p, 4,
                                              ctypes.c_float(0.1), bs, ctypes.byref(d))
        return rc, launches() - n0

    ok_slots = list(range(20, 23)) + list(range(40, 49))
    expect("debug prefill step: valid launches once", prefill_step_with([0, 3, 12], ok_slots),
           (_lib.PA_OK, 1))
    expect("debug prefill step: duplicate slot",
           prefill_step_with([0, 3, 12], ok_slots[:-1] + [20]), (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug prefill step: slot past the pool",
           prefill_step_with([0, 3, 12], ok_slots[:-1] + [nb * bs]),
           (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug prefill step: bad query_start",
           prefill_step_with([0, 13, 12], ok_slots), (_lib.PA_ERR_PRECONDITION, 0))

    # page copies
    def copy_with(pairs, same_pool):
        flat = [x for pr in pairs for x in pr]
        m, m_p = _arr(ctypes.c_int64, flat)
        d = _lib.CopyDims()
        d.num_pairs, d.num_kv_heads, d.head_dim, d.block_size = len(pairs), 8, 128, 16
        d.dtype, d.src_num_blocks, d.dst_num_blocks = _lib.PA_DTYPE_BF16, nb, nb
        dst = (P, P) if same_pool else (P + 4096, P + 8192)
        n0 = launches()
        rc = lib.copy_blocks(P, P, dst[0], dst[1], m_p, ctypes.byref(d))
        return rc, launches() - n0

    expect("debug: valid copies", copy_with([(1, 2), (3, 4), (-1, 2), (5, nb)], True),
           (_lib.PA_OK, 1))
    expect("debug: repeated destination", copy_with([(1, 2), (3, 2)], False),
           (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: destination is a source in one pool", copy_with([(1, 2), (2, 4)], True),
           (_lib.PA_ERR_PRECONDITION, 0))
    expect("debug: chains are fine across pools", copy_with([(1, 2), (2, 4)], False),
           (_lib.PA_OK, 1))
    os.environ.pop("PA_DEBUG_CHECKS", None)
