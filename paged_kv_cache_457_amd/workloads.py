"""Seeded synthetic inputs for paged decode attention and the KV-cache write.

This module only *builds inputs*: a physical page pool, per-sequence block
tables, context lengths, queries, the new token's K/V and the slot each new
token is written to.  It plays the part of the page manager that the pages put
in front of the attention kernel (vLLM / PagedAttention pages: the page pool
with its allocate-on-arrival lifecycle, and the page-table figure in the
PagedAttention section of the tutorial page, chapter 4.2): pages are handed out
from a shuffled free list, so a sequence's logical pages sit at scattered
physical pages.  It computes no attention, no softmax and no cache write; the
HIP library and the CPU oracle both consume the arrays built here.

Conventions (shared by both sides, so fixed here once):

* pools ``k_pool`` / ``v_pool`` have shape ``[num_blocks, num_kv_heads,
  block_size, head_dim]``; token ``t`` of a sequence lives in logical page
  ``t // block_size`` at offset ``t % block_size``;
* ``context_lens[s]`` counts every token attention reads for sequence ``s``,
  *including* the token appended in the same decode step; the pools returned
  here hold the state *before* that append (``ctx - 1`` live tokens) and the
  append goes to ``slot_mapping[s] = page * block_size + offset`` of position
  ``ctx - 1``;
* every pool slot that holds no live token is poisoned with NaN, so a kernel
  that lets a masked or unused slot reach its arithmetic shows NaN;
* block-table columns past ``ceil(ctx / block_size)`` hold ``-1``;
* bf16 values are stored as raw ``uint16`` bit patterns, rounded from fp32
  draws with round-to-nearest-even; fp32 values are ``float32``.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)
UNUSED_TABLE_ENTRY = np.int32(-1)

# Draw chunk for the bulk N(0,1) fill.  Every chunk has its own child seed, so
# the values do not depend on how many threads fill them.
_CHUNK = 1 << 22


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def storage_dtype(dtype: str):
    if dtype == "f32":
        return np.float32
    if dtype == "bf16":
        return np.uint16
    raise ValueError(f"unsupported dtype {dtype!r}")


def nan_value(dtype: str):
    return np.float32(np.nan) if dtype == "f32" else BF16_NAN_BITS


def _normal_fill(seed_seq: np.random.SeedSequence, n: int, dtype: str,
                 threads: Optional[int] = None) -> np.ndarray:
    """n draws of N(0,1) in the storage dtype, chunked with per-chunk seeds."""
    out = np.empty(n, dtype=storage_dtype(dtype))
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = seed_seq.spawn(nchunks)

    def fill(i: int) -> None:
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        if lo >= hi:
            return
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else round_f32_to_bf16_bits(x)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nchunks == 1 or threads <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


@dataclass
class Workload:
    """One decode step's inputs; see the module docstring for conventions."""
    name: str
    dtype: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    refcount: np.ndarray
    seed: int
    extra: Dict[str, object] = field(default_factory=dict)
    # split-K partition size the configuration names, in tokens (0: the
    # library's default)
    partition_size: int = 0
    # multi-token steps (prefill): rows of q / k_new / v_new / slot_mapping
    # of sequence s are query_start[s] .. query_start[s+1]-1; None for a
    # decode step (one row per sequence)
    query_start: Optional[np.ndarray] = None

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def kv_bytes(self) -> int:
        """KV bytes one decode call reads: sum ctx * Hkv * D * 2 * sizeof."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads \
            * self.head_dim * 2 * self.elem_bytes

    @property
    def num_tokens(self) -> int:
        return int(self.q.shape[0])

    def prefill_flops(self) -> int:
        """Multiply-add flops of a prefill step: every chunk row at position p
        costs 2 * D (q . K) + 2 * D (P . V) per visible token (p + 1 of them),
        for each of the H query heads."""
        assert self.query_start is not None
        n = np.diff(self.query_start.astype(np.int64))
        ctx = self.context_lens.astype(np.int64)
        # sum over i < n of (ctx - n + i + 1) = n * (ctx - n) + n (n + 1) / 2
        visible = n * (ctx - n) + n * (n + 1) // 2
        return int(visible.sum()) * 4 * self.head_dim * self.num_heads

    def unique_kv_bytes(self) -> int:
        """KV bytes counting each physical (page, slot) once (shared prefixes)."""
        bs = self.block_size
        seen = set()
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for j in range((L + bs - 1) // bs):
                n = min(bs, L - j * bs)
                seen.add((int(self.block_tables[s, j]), n))
        per_page = {}
        for b, n in seen:
            per_page[b] = max(per_page.get(b, 0), n)
        toks = sum(per_page.values())
        return toks * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes


def _page_counts(ctx: np.ndarray, bs: int) -> np.ndarray:
    return (ctx.astype(np.int64) + bs - 1) // bs


def build_workload(name: str, ctx: Sequence[int], num_heads: int, num_kv_heads: int,
                   head_dim: int, block_size: int, dtype: str, seed: int,
                   num_blocks: Optional[int] = None, pool_factor: float = 1.25,
                   max_blocks_per_seq: Optional[int] = None,
                   shared_prefix: Optional[List[List[int]]] = None,
                   shared_prefix_len: int = 0,
                   poison: bool = True,
                   rng: Optional[np.random.Generator] = None,
                   new_tokens: Optional[Sequence[int]] = None) -> Workload:
    """Allocate pages for ``ctx`` tokens per sequence and fill the pool.

    ``shared_prefix`` lists groups of sequence indices whose first
    ``shared_prefix_len`` tokens (a whole number of pages) sit on the same
    physical pages, the parallel-sampling sharing of the tutorial page's 4.2;
    those pages carry a reference count equal to the group size.  The token
    appended in this step always lands on a page the sequence owns alone.

    ``new_tokens`` makes it a multi-token step (a prefill chunk): sequence s
    appends its last ``new_tokens[s]`` tokens in this step, so the pools hold
    ``ctx - new_tokens`` live tokens, q / k_new / v_new / slot_mapping have
    one row per appended token, packed by sequence, and ``query_start``
    gives each sequence's first row.  Without it each sequence appends one
    token (none when ctx == 0) and has one row.
    """
    ctx = np.asarray(ctx, dtype=np.int64)
    S = len(ctx)
    if num_heads % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if np.any(ctx < 0):
        raise ValueError("negative context length")
    bs = block_size
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    pages = _page_counts(ctx, bs)
    shared_pages_per_seq = np.zeros(S, dtype=np.int64)
    groups = shared_prefix or []
    if groups:
        if shared_prefix_len % bs:
            raise ValueError("a shared prefix must be a whole number of pages")
        npp = shared_prefix_len // bs
        for grp in groups:
            for s in grp:
                if ctx[s] <= shared_prefix_len:
                    raise ValueError("the appended token must fall past the shared prefix")
                shared_pages_per_seq[s] = npp
    private_pages = pages - shared_pages_per_seq
    needed = int(private_pages.sum()) + len(groups) * (shared_prefix_len // bs if groups else 0)
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * needed)))
    if needed > num_blocks:
        raise ValueError(f"pool of {num_blocks} pages cannot hold {needed}")
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(pages.max()) if S else 1)
    if S and int(pages.max()) > max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq too small for the longest sequence")

    # free list: a random permutation of the physical pages, taken in order
    free = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    bt = np.full((S, max_blocks_per_seq), UNUSED_TABLE_ENTRY, dtype=np.int32)
    refcount = np.zeros(num_blocks, dtype=np.int32)
    for grp in groups:
        npp = shared_prefix_len // bs
        shared = free[cursor:cursor + npp]
        cursor += npp
        for s in grp:
            bt[s, :npp] = shared
        refcount[shared] += len(grp)
    for s in range(S):
        lo = int(shared_pages_per_seq[s])
        n = int(pages[s]) - lo
        own = free[cursor:cursor + n]
        cursor += n
        bt[s, lo:lo + n] = own
        refcount[own] += 1

    # tokens appended in this step, per sequence
    if new_tokens is None:
        appended = np.minimum(ctx, 1)
    else:
        appended = np.asarray(new_tokens, dtype=np.int64)
        if appended.shape != (S,) or np.any(appended < 0) or np.any(appended > ctx):
            raise ValueError("new_tokens must be between 0 and the context length")

    # live slots of the pre-append state: positions 0 .. ctx - appended - 1
    live = np.zeros((num_blocks, bs), dtype=bool)
    for s in range(S):
        L = int(ctx[s] - appended[s])
        if L <= 0:
            continue
        full = L // bs
        if full:
            live[bt[s, :full], :] = True
        rem = L - full * bs
        if rem:
            live[bt[s, full], :rem] = True

    # slots of the appended positions ctx - appended .. ctx - 1; a decode
    # step keeps one row per sequence (slot -1 when ctx == 0)
    if new_tokens is None:
        query_start = None
        slot = np.full(S, -1, dtype=np.int64)
        for s in range(S):
            if ctx[s] >= 1:
                pos = int(ctx[s]) - 1
                slot[s] = int(bt[s, pos // bs]) * bs + pos % bs
    else:
        query_start = np.concatenate([[0], np.cumsum(appended)]).astype(np.int32)
        slot = np.full(int(appended.sum()), -1, dtype=np.int64)
        for s in range(S):
            for i in range(int(appended[s])):
                pos = int(ctx[s] - appended[s]) + i
                slot[query_start[s] + i] = int(bt[s, pos // bs]) * bs + pos % bs
    if S and len(set(slot[slot >= 0].tolist())) != int((slot >= 0).sum()):
        raise AssertionError("new-token slots collide")
    for s in range(S):
        if slot[s] >= 0 and refcount[slot[s] // bs] != 1:
            raise AssertionError("append would land on a shared page")

    H, Hkv, D = num_heads, num_kv_heads, head_dim
    ss = np.random.SeedSequence([seed, 457])
    k_ss, v_ss, q_ss, kn_ss, vn_ss = ss.spawn(5)
    pool_shape = (num_blocks, Hkv, bs, D)
    pool_n = int(np.prod(pool_shape))
    k_pool = _normal_fill(k_ss, pool_n, dtype).reshape(pool_shape)
    v_pool = _normal_fill(v_ss, pool_n, dtype).reshape(pool_shape)
    if poison:
        dead_b, dead_o = np.nonzero(~live)
        nanv = nan_value(dtype)
        k_pool[dead_b, :, dead_o, :] = nanv
        v_pool[dead_b, :, dead_o, :] = nanv
    T = len(slot)
    q = _normal_fill(q_ss, T * H * D, dtype).reshape(T, H, D)
    k_new = _normal_fill(kn_ss, T * Hkv * D, dtype).reshape(T, Hkv, D)
    v_new = _normal_fill(vn_ss, T * Hkv * D, dtype).reshape(T, Hkv, D)

    return Workload(
        name=name, dtype=dtype, num_seqs=S, num_heads=H, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, num_blocks=num_blocks,
        max_blocks_per_seq=max_blocks_per_seq,
        scale=np.float32(1.0 / math.sqrt(D)), q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=bt, context_lens=ctx.astype(np.int32), k_new=k_new,
        v_new=v_new, slot_mapping=slot, refcount=refcount, seed=seed,
        extra={"live": live}, query_start=query_start)


def free_slots(w: Workload, count: int, rng: np.random.Generator) -> np.ndarray:
    """``count`` distinct slots that hold no live token and are not this
    step's append slots: the "random free slots" of the tiny configuration."""
    live = w.extra["live"].copy()
    for sl in w.slot_mapping:
        if sl >= 0:
            live[sl // w.block_size, sl % w.block_size] = True
    cand = np.flatnonzero(~live.reshape(-1))
    pick = rng.choice(cand, size=count, replace=False)
    return pick.astype(np.int64)


CONFIG_NAMES = {
    1: "tiny paged decode (4 seqs, ctx {1,17,33,100}, 4/4 heads, D 64, bs 16, fp32)",
    2: "Llama-2-7B decode (64 seqs, ctx U[128,2048], 32/32 heads, D 128, bs 16, bf16)",
    3: "GQA high batch (256 seqs, ctx lognormal med 512 s1 [16,8192], 32/8 heads, D 128, bs 16, bf16)",
    4: "long-context split-K (8 seqs x 32768, 32/8 heads, D 128, bs 32, bf16)",
    5: "prefix-shared sampling (16 prompts x 8 samples, 1024 shared + U[0,256] + 1, 32/8 heads, D 128, bs 16, bf16)",
}

DEFAULT_SEED_BASE = 4570


def make_config(index: int, seed: Optional[int] = None) -> Workload:
    """The five workload configurations, by number (1..5)."""
    if seed is None:
        seed = DEFAULT_SEED_BASE + index
    rng = np.random.Generator(np.random.PCG64(seed))
    if index == 1:
        w = build_workload("c1", [1, 17, 33, 100], 4, 4, 64, 16, "f32", seed,
                           num_blocks=64, rng=rng)
        w.extra["free_slots"] = free_slots(w, 4, rng)
        w.extra["free_k"] = _normal_fill(np.random.SeedSequence([seed, 1]),
                                         4 * 4 * 64, "f32").reshape(4, 4, 64)
        w.extra["free_v"] = _normal_fill(np.random.SeedSequence([seed, 2]),
                                         4 * 4 * 64, "f32").reshape(4, 4, 64)
        return w
    if index == 2:
        ctx = rng.integers(128, 2048, size=64, endpoint=True)
        return build_workload("c2", ctx, 32, 32, 128, 16, "bf16", seed,
                              max_blocks_per_seq=2048 // 16, rng=rng)
    if index == 3:
        z = rng.standard_normal(256)
        ctx = np.clip(np.rint(512.0 * np.exp(z)), 16, 8192).astype(np.int64)
        return build_workload("c3", ctx, 32, 8, 128, 16, "bf16", seed,
                              max_blocks_per_seq=8192 // 16, rng=rng)
    if index == 4:
        ctx = np.full(8, 32768, dtype=np.int64)
        w = build_workload("c4", ctx, 32, 8, 128, 32, "bf16", seed,
                           max_blocks_per_seq=32768 // 32, rng=rng)
        w.partition_size = 512
        return w
    if index == 5:
        prompts, samples, prefix = 16, 8, 1024
        div = rng.integers(0, 256, size=(prompts, samples), endpoint=True)
        # sample 0 of each prompt appends exactly on a page boundary
        div[:, 0] = 16 * rng.integers(0, 16, size=prompts, endpoint=True)
        ctx = (prefix + div + 1).reshape(-1)
        groups = [list(range(p * samples, (p + 1) * samples)) for p in range(prompts)]
        w = build_workload("c5", ctx, 32, 8, 128, 16, "bf16", seed,
                           max_blocks_per_seq=(prefix + 256 + 1 + 15) // 16,
                           shared_prefix=groups, shared_prefix_len=prefix, rng=rng)
        w.extra["divergent"] = div.reshape(-1)
        # the sharing structure, for the shared-prefix decode entry point
        w.extra["group_starts"] = np.arange(0, prompts * samples + 1, samples, dtype=np.int32)
        w.extra["prefix_lens"] = np.full(prompts, prefix, dtype=np.int32)
        return w
    raise ValueError(f"no configuration {index}")


PREFILL_CONFIG_NAMES = {
    1: "tiny prefill (4 seqs, cached {0,5,16,40} + new {1,12,33,7}, 4/2 heads, D 64, bs 16, bf16)",
    2: "Llama-2-7B chunked prefill (8 seqs, 1024 new after U[0,3072] cached, 32/32 heads, D 128, bs 16, bf16)",
    3: "GQA prompt prefill (16 prompts U[256,2048], nothing cached, 32/8 heads, D 128, bs 16, bf16)",
    4: "long-context chunked prefill (2 seqs: 512 new after 15872 cached, 256 new after 7680 "
       "cached; 32/8 heads, D 128, bs 16, bf16)",
}

PREFILL_SEED_BASE = 4580


def make_prefill_config(index: int, seed: Optional[int] = None) -> Workload:
    """Multi-token (prefill) steps, by number (1..4): newly admitted requests
    whose prompt, or a chunk of it, is appended and attended in one step."""
    if seed is None:
        seed = PREFILL_SEED_BASE + index
    rng = np.random.Generator(np.random.PCG64(seed))
    if index == 1:
        cached, new = np.array([0, 5, 16, 40]), np.array([1, 12, 33, 7])
        return build_workload("p1", cached + new, 4, 2, 64, 16, "bf16", seed, rng=rng,
                              new_tokens=new)
    if index == 2:
        cached = rng.integers(0, 3072, size=8, endpoint=True)
        new = np.full(8, 1024)
        return build_workload("p2", cached + new, 32, 32, 128, 16, "bf16", seed,
                              max_blocks_per_seq=(3072 + 1024) // 16, rng=rng, new_tokens=new)
    if index == 3:
        new = rng.integers(256, 2048, size=16, endpoint=True)
        return build_workload("p3", new, 32, 8, 128, 16, "bf16", seed,
                              max_blocks_per_seq=2048 // 16, rng=rng, new_tokens=new)
    if index == 4:
        # the next chunk of two long prompts: few query rows over many cached keys
        cached, new = np.array([15872, 7680]), np.array([512, 256])
        return build_workload("p4", cached + new, 32, 8, 128, 16, "bf16", seed,
                              max_blocks_per_seq=16384 // 16, rng=rng, new_tokens=new)
    raise ValueError(f"no prefill configuration {index}")
