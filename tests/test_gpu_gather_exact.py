"""Bit-exact block-table indexing at full size, on every decode kernel form.

A peaked softmax has a unique exact answer.  With q = 8 e0 on every query
head and K[t][0] = 0 on every slot, every logit is exactly 0; one target
token t* per (sequence, kv-head) gets K[t*][0] = 256, so its logit is
8 * 256 * scale (181 at head_dim 128, 256 at 64) above all others.  Every
other weight, exp(-181) and below, is 0 in fp32 -- inside a partition and
across the log-sum-exp merge of partitions -- and the output rows of that
kv-head's query heads must equal the target's V row bit for bit.  A K row
read from a wrong page or slot moves the peak (the output becomes a mean);
a V row read from a wrong place changes the bits.

Each call places one target per (sequence, kv-head), edited on the device
in the pool the cache write filled, and restores it after the call.  The
calls sweep every page of every sequence, rotating the slot among the
first, an interior and the last live slot of the page, plus every
partition edge (both sides), the first token, the last two tokens and the
appended token.  Expected rows come from the host pools after the oracle's
cache write, never from the device.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_457_amd import binding
from paged_kv_cache_457_amd.device_inputs import to_host, upload
from paged_kv_cache_457_amd.workloads import build_workload, make_config

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _prepare(w):
    """Device inputs after the step's cache write with every logit made 0,
    and the host pools after the same write (for the expected rows)."""
    dw = upload(w)
    binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool, dw.slot_mapping)
    kp, vp = oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool, w.slot_mapping,
                                      w.block_size)
    del kp
    dw.q.zero_()
    dw.q[:, :, 0] = 8.0
    dw.k_pool[:, :, :, 0] = 0
    torch.cuda.synchronize()
    return dw, vp


def _slot_in_page(w, s, j, cls, salt):
    """Slot class cls (0 first, 1 last live, 2 interior) of logical page j
    of sequence s."""
    bs = w.block_size
    n = min(bs, int(w.context_lens[s]) - j * bs)       # live slots of the page
    if cls == 0 or n == 1:
        return 0
    if cls == 1 or n == 2:
        return n - 1
    return 1 + salt % (n - 2)


def page_sweep(w, members=None):
    """Calls (lists of (s, g, t)) that together put a target on every page
    of every sequence, rotating the slot class; `members` restricts the
    sequences (default all)."""
    S, hkv, bs = w.num_seqs, w.num_kv_heads, w.block_size
    seqs = list(range(S)) if members is None else members
    npages = {s: -(-int(w.context_lens[s]) // bs) for s in seqs}
    top = max([n for n in npages.values()] + [0])
    calls = []
    for c in range(-(-top // hkv)):
        tg = []
        for s in seqs:
            if npages[s] == 0:
                continue
            for g in range(hkv):
                j = (c * hkv + g + s) % npages[s]
                off = _slot_in_page(w, s, j, (c + g + s) % 3, 7 * c + 3 * g + s)
                tg.append((s, g, j * bs + off))
        calls.append(tg)
    return calls


def edge_calls(w, part_tokens, members=None, extra=()):
    """Calls that target, for each sequence, token 0, the last two tokens,
    both sides of every partition edge and any `extra` positions."""
    hkv = w.num_kv_heads
    seqs = list(range(w.num_seqs)) if members is None else members
    want = {}
    for s in seqs:
        L = int(w.context_lens[s])
        if L == 0:
            continue
        ts = {0, L - 1, max(L - 2, 0)} | {t for t in extra if 0 <= t < L}
        for e in range(part_tokens, L, part_tokens):
            ts |= {e - 1, e}
        want[s] = sorted(ts)
    calls = []
    for c in range(-(-max([len(v) for v in want.values()] + [0]) // hkv)):
        tg = [(s, g, ts[c * hkv + g]) for s, ts in want.items() for g in range(hkv)
              if c * hkv + g < len(ts)]
        calls.append(tg)
    return calls


BIG = {"bf16": 256.0, "f32": 256.0}


def run_targets(w, dw, vp, calls, decode, expect_rows=None):
    """Run each call with its targets raised; check the rows bit for bit.
    `expect_rows(s, g, t)` lists the sequences whose kv-head g rows must
    equal the target's V row (default: s alone)."""
    bs, G = w.block_size, w.group
    bt = w.block_tables
    checked = 0
    for tg in calls:
        if not tg:
            continue
        dev = dw.k_pool.device
        pages = torch.tensor([int(bt[s, t // bs]) for s, g, t in tg], device=dev)
        heads = torch.tensor([g for _, g, _ in tg], device=dev)
        offs = torch.tensor([t % bs for _, _, t in tg], device=dev)
        dw.k_pool[pages, heads, offs, 0] = BIG[w.dtype]
        decode(dw)
        if dev.type == "cuda":
            torch.cuda.synchronize()
        got = to_host(dw.out, w.dtype)
        dw.k_pool[pages, heads, offs, 0] = 0
        for s, g, t in tg:
            row = vp[bt[s, t // bs], g, t % bs].tobytes()
            for m in (expect_rows(s, g, t) if expect_rows else [s]):
                for h in range(g * G, (g + 1) * G):
                    assert got[m, h].tobytes() == row, (m, h, s, g, t)
                    checked += 1
    return checked


def plain_decode(partition_size):
    def call(dw):
        binding.paged_attention_decode(dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables,
                                       dw.context_lens, scale=float(dw.w.scale),
                                       partition_size=partition_size)
    return call


def _sweep_plain(w, partition_size, label):
    dw, vp = _prepare(w)
    part = binding.paged_attention_decode_partition_tokens(dw.q, dw.k_pool, dw.block_tables,
                                                           partition_size)
    parts = -(-w.max_blocks_per_seq * w.block_size // part)
    calls = page_sweep(w) + edge_calls(w, part)
    say(f"{label}: {w.num_seqs} x {w.num_kv_heads} kv-heads, partition {part} tokens "
        f"({parts} per full table), {len(calls)} calls")
    n = run_targets(w, dw, vp, calls, plain_decode(partition_size))
    say(f"  {n} rows bit-exact")


@functools.lru_cache(maxsize=1)
def _config(i):
    """The configuration's inputs, generated once for consecutive tests."""
    return make_config(i)


def test_long_context_one_wave_gqa_bit_exact():
    """8 x 32768 tokens, 32/8 heads, 32-token pages, 512-token partitions:
    64 partitions per sequence, the grouped-query kernel's one-wave-per-item
    form and the 64-way log-sum-exp merge."""
    _sweep_plain(_config(4), 512, "c4 shape")


def test_long_context_default_partition_bit_exact():
    """The same batch at the library's default partition (2048 tokens:
    16 partitions, still one wave per item)."""
    _sweep_plain(_config(4), 0, "c4 shape, default partition")


@pytest.mark.parametrize("ps", [0, 128])
def test_mha_valu_bit_exact(ps):
    """The Llama-2-7B shape (64 sequences, 32/32 heads, 16-token pages) on the
    VALU kernel: one partition per sequence (default) and 128-token
    partitions (16 per full table, eight-wave items, the many-partials
    merge)."""
    _sweep_plain(_config(2), ps, f"c2 shape, partition {ps}")


def test_ragged_gqa_four_wave_bit_exact():
    """256 lognormal sequences, 32/8 heads at the default 2048-token
    partition: the grouped-query kernel's four-wave items, up to 4
    partitions, the few-partials merge."""
    _sweep_plain(_config(3), 0, "c3 shape")


def test_fp32_many_partitions_bit_exact():
    """fp32 with two query heads per kv-head (VALU), 256-token partitions:
    16 per full table, ragged lengths."""
    ctx = [4096, 4095, 3001, 2048, 513, 512, 17, 1, 0, 4000]
    w = build_workload("peak-f32", ctx, 16, 8, 128, 16, "f32", seed=91, max_blocks_per_seq=256)
    _sweep_plain(w, 256, "fp32 G2")


VARIANTS = [(dt, D, bs, G) for dt in ("f32", "bf16") for D in (64, 128) for bs in (16, 32)
            for G in (1, 2, 4, 8)]


@pytest.mark.parametrize("dt,D,bs,G", VARIANTS, ids=[f"{a}-D{b}-bs{c}-G{d}" for a, b, c, d in VARIANTS])
def test_every_variant_many_partitions_bit_exact(dt, D, bs, G):
    """Every built variant with four-page partitions over a 2048-token
    table (16 or 32 partitions: the one-wave grouped-query form for bf16
    with a head group) and a whole-table partition."""
    ctx = [2048, 2047, 1000, 4 * bs + 1, 4 * bs, bs, 3, 0]
    w = build_workload("peak-var", ctx, 8 * G, 8, D, bs, dt, seed=300 + D + bs + G,
                       max_blocks_per_seq=2048 // bs)
    for ps in (4 * bs, 0):
        _sweep_plain(w, ps, f"{dt} D{D} bs{bs} G{G} partition {ps}")


# ---------------------------------------------------------- shared prefixes
def shared_decode(starts, prefixes, partition_size):
    def call(dw):
        binding.paged_attention_decode_shared_prefix(
            dw.out, dw.q, dw.k_pool, dw.v_pool, dw.block_tables, dw.context_lens,
            torch.tensor(starts, dtype=torch.int32, device="cuda"),
            torch.tensor(prefixes, dtype=torch.int32, device="cuda"),
            scale=float(dw.w.scale), partition_size=partition_size)
    return call


def _sweep_shared(w, groups, prefix_len, partition_size, label):
    """Prefix targets (one per group and kv-head, on a shared page: every
    member's rows must show it), then own-page targets (one per member and
    kv-head)."""
    bs, hkv = w.block_size, w.num_kv_heads
    npp = prefix_len // bs
    starts = [0]
    for g in groups:
        starts.append(starts[-1] + len(g))
    dw, vp = _prepare(w)
    call = shared_decode(starts, [prefix_len] * len(groups), partition_size)
    part = partition_size or min(512, w.max_blocks_per_seq * bs)
    member_of = {s: grp for grp in groups for s in grp}
    # prefix: pages 0 .. npp - 1 through the group's first member
    pre_calls = []
    for c in range(-(-npp // hkv)):
        tg = []
        for gi, grp in enumerate(groups):
            for g in range(hkv):
                j = (c * hkv + g + gi) % npp
                off = (0, bs - 1, 1 + (7 * c + g) % (bs - 2))[(c + g + gi) % 3]
                tg.append((grp[0], g, j * bs + off))
        pre_calls.append(tg)
    edges = sorted({t for e in range(part, prefix_len + 1, part) for t in (e - 1, e)
                    if t < prefix_len} | {0, prefix_len - 1})
    for c in range(-(-len(edges) // hkv)):
        pre_calls.append([(grp[0], g, edges[c * hkv + g]) for grp in groups for g in range(hkv)
                          if c * hkv + g < len(edges)])
    n = run_targets(w, dw, vp, pre_calls, call, expect_rows=lambda s, g, t: member_of[s])
    # own pages: each member's pages from npp on, every page and the edges
    own_calls = []
    owns = {s: list(range(npp, -(-int(w.context_lens[s]) // bs))) for s in member_of}
    top = max(len(v) for v in owns.values())
    for c in range(-(-top // hkv)):
        tg = []
        for s, pages in owns.items():
            for g in range(hkv):
                j = pages[(c * hkv + g + s) % len(pages)]
                off = _slot_in_page(w, s, j, (c + g + s) % 3, 5 * c + g)
                tg.append((s, g, j * bs + off))
        own_calls.append(tg)
    own_calls += edge_calls(w, part, members=list(member_of), extra=(prefix_len,))
    # edge_calls also targets tokens inside the prefix (token 0, partition
    # edges): those pages are shared, so only own-page targets stay here
    own_calls = [[(s, g, t) for s, g, t in tg if t >= prefix_len] for tg in own_calls]
    n += run_targets(w, dw, vp, own_calls, call)
    say(f"{label}: {len(pre_calls)} prefix calls, {len(own_calls)} own-page calls, "
        f"{n} rows bit-exact")


def test_shared_prefix_c5_bit_exact():
    """16 prompts x 8 samples sharing a 1024-token prefix (64 pages), 32/8
    heads: 32 query rows per prefix unit (two row tiles)."""
    w = _config(5)
    starts = w.extra["group_starts"]
    groups = [list(range(starts[i], starts[i + 1])) for i in range(len(starts) - 1)]
    _sweep_shared(w, groups, int(w.extra["prefix_lens"][0]), 0, "c5 shared prefix")


def test_shared_prefix_over_128_pages_two_tiles_bit_exact():
    """A 3200-token prefix (200 pages) in one 256-page partition, six members
    x 4 query heads = 24 rows: two row tiles, two waves per tile, so each
    wave takes up to 100 of the unit's pages -- more than one page id per
    lane."""
    rng = np.random.default_rng(77)
    bs, prefix, members = 16, 3200, 6
    own = rng.integers(0, 40, size=members)
    ctx = [prefix + int(o) + 1 for o in own]
    mb = -(-max(ctx) // bs)
    w = build_workload("sp-long", ctx, 16, 4, 128, bs, "bf16", seed=78, max_blocks_per_seq=mb,
                       shared_prefix=[list(range(members))], shared_prefix_len=prefix)
    # a plain tolerance check against the oracle first
    ref = oracle.decode(w.q, *oracle.reshape_and_cache(w.k_new, w.v_new, w.k_pool, w.v_pool,
                                                       w.slot_mapping, bs),
                        w.block_tables, w.context_lens, w.num_kv_heads, w.scale, bs, "bf16")
    dw = upload(w)
    binding.reshape_and_cache(dw.k_new, dw.v_new, dw.k_pool, dw.v_pool, dw.slot_mapping)
    shared_decode([0, members], [prefix], 256 * bs)(dw)
    torch.cuda.synchronize()
    err = float(np.max(np.abs(oracle.widen(to_host(dw.out, "bf16"), "bf16") - ref)))
    say(f"200-page prefix, 256-page partition: max abs err {err:.3e}")
    assert err <= 1e-2
    del dw
    _sweep_shared(w, [list(range(members))], prefix, 256 * bs, "200-page prefix, two tiles")
