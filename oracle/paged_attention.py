"""CPU oracle for paged decode and prefill attention, the KV-cache write and
the page copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg call it.
It shares no code with the HIP library: no kernels, headers, helpers or
constants.  It is plain, slow and written to be checked by eye.

What it computes (vLLM / PagedAttention pages):

* The showapi.com article, section 2.1, and the tutorial page, chapter 4.2,
  say that paging changes only *where* the KV cache lives: the cache is cut
  into fixed-size pages, a per-request page table maps logical pages to
  physical pages, and the attention kernel reads the pages through that table
  with no data movement and no padding.  So decode attention over a paged
  cache is ordinary single-query softmax attention over the sequence's tokens
  in logical order; the only paged part is the gather.  ``decode`` walks each
  sequence's logical pages in order, looks each up in the block table, reads
  that page's tokens, and then applies softmax(q . K^T * scale) . V per head.
* ``prefill`` is the same attention for several new tokens of a sequence at
  once (a newly admitted request's prompt, or a chunk of it; tutorial page,
  chapter 4.3, step 2), each token attending causally to the tokens up to
  its own position.
* The tutorial page, chapter 4.3 (step 3 of the iteration), says each forward
  step yields the next token together with the updated KV cache.
  ``reshape_and_cache`` is that update: every new token's K and V rows go to
  the pool slot named by its slot number, ``slot = physical_page * block_size
  + offset``.

Readings where the pages are silent (the attention formula, the scale, the
GQA head map, the pool layout, ctx == 0, duplicate slots) are stated at each
function.  Arithmetic is float64; bf16 inputs are widened exactly.
"""
from __future__ import annotations

import numpy as np

__all__ = ["widen", "gather_pages", "decode", "prefill", "rope", "reshape_and_cache", "copy_blocks"]


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64.

    ``dtype == "bf16"``: ``x`` holds raw 16-bit patterns; a bfloat16 is the
    top half of an IEEE binary32, so placing the 16 bits in the high half of a
    32-bit word gives the same value as a float32, which widens exactly.
    ``dtype == "f32"``: float32 widens exactly.
    """
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unsupported dtype {dtype!r}")


def gather_pages(pool: np.ndarray, table_row: np.ndarray, ctx: int,
                 block_size: int) -> np.ndarray:
    """Tokens 0..ctx-1 of one sequence, in logical order, as [Hkv, ctx, D].

    Logical page j of the sequence is physical page ``table_row[j]``; token t
    lives in logical page t // block_size at offset t % block_size (pages fill
    in token order: the page table keeps the logical view contiguous while the
    physical pages are scattered, tutorial page 4.2).  Only the first
    ceil(ctx / block_size) table entries are read.
    """
    num_blocks, hkv, bs, d = pool.shape
    assert bs == block_size
    pieces = []
    npages = (ctx + block_size - 1) // block_size
    for j in range(npages):
        phys = int(table_row[j])
        if not 0 <= phys < num_blocks:
            raise IndexError(f"logical page {j} maps to physical page {phys}, "
                             f"outside the pool of {num_blocks}")
        n = min(block_size, ctx - j * block_size)
        pieces.append(pool[phys, :, :n, :])
    if not pieces:
        return np.zeros((hkv, 0, d), dtype=pool.dtype)
    return np.concatenate(pieces, axis=1)


def decode(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
           block_tables: np.ndarray, context_lens: np.ndarray,
           num_kv_heads: int, scale, block_size: int, dtype: str,
           return_lse: bool = False, alibi_slopes=None):
    """Single-token decode attention over a paged KV cache, in float64.

    q            [S, H, D]          stored values (float32, or bf16 bits)
    k_pool       [NB, Hkv, bs, D]   same
    v_pool       [NB, Hkv, bs, D]   same
    block_tables [S, max_blocks]    int, logical page -> physical page
    context_lens [S]                tokens attended per sequence

    Readings: out[s, h] = softmax(scale * K q[s, h]) V over the sequence's
    ctx tokens, with the safe-softmax max subtracted (mathematically the same
    result).  ``scale`` is used at the exact float32 value the GPU receives.
    Query head h reads kv-head h // (H / Hkv): consecutive q heads form a
    group (grouped-query attention).  ctx == 0 gives a zero row (and
    lse = -inf).  Returns out [S, H, D] float64, and with ``return_lse`` also
    the log-sum-exp of the scaled logits [S, H].

    ``alibi_slopes`` (optional, [H]): the ALiBi model variant (showapi.com
    article, section 4.1, names ALiBi among the position encodings the
    engine serves).  Reading: the logit of token t gets slope_h * (t - p)
    added, p = ctx - 1 being the query's own position, so nearer tokens
    weigh more for a positive slope.  Slopes are used at their float32
    values.
    """
    S, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("H must be a multiple of num_kv_heads")
    group = H // num_kv_heads
    sc = float(np.float32(scale))
    out = np.zeros((S, H, D), dtype=np.float64)
    lse = np.full((S, H), -np.inf, dtype=np.float64)
    qf = widen(q, dtype)
    for s in range(S):
        L = int(context_lens[s])
        if L < 0:
            raise ValueError("negative context length")
        if L == 0:
            continue
        if (L + block_size - 1) // block_size > block_tables.shape[1]:
            raise ValueError("context longer than the block table")
        K = widen(gather_pages(k_pool, block_tables[s], L, block_size), dtype)
        V = widen(gather_pages(v_pool, block_tables[s], L, block_size), dtype)
        for h in range(H):
            g = h // group
            logits = sc * (K[g] @ qf[s, h])              # [L]
            if alibi_slopes is not None:
                logits = logits + float(np.float32(alibi_slopes[h])) * (np.arange(L) - (L - 1))
            m = logits.max()
            p = np.exp(logits - m)
            z = p.sum()
            out[s, h] = (p @ V[g]) / z
            lse[s, h] = m + np.log(z)
    if return_lse:
        return out, lse
    return out


def prefill(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
            block_tables: np.ndarray, context_lens: np.ndarray,
            query_start: np.ndarray, num_kv_heads: int, scale, block_size: int,
            dtype: str, rows=None, alibi_slopes=None) -> np.ndarray:
    """Multi-token attention over a paged KV cache (prefill and chunked
    prefill), in float64.

    q            [T, H, D]        the new tokens of all sequences, packed:
                                  sequence s owns rows query_start[s] ..
                                  query_start[s + 1] - 1
    query_start  [S + 1]          int, 0 = query_start[0] <= ... <= query_start[S] = T
    context_lens [S]              tokens of sequence s in the cache once this
                                  chunk is written (earlier tokens + chunk)
    pools, block_tables           as for ``decode``; the chunk's own K/V rows
                                  are already in the pool (the cache write
                                  of the same step)

    Where it comes from: continuous batching admits a new request into the
    running batch at the next iteration, with pages allocated for it
    (tutorial page, section 4.3, steps 2-3; pinggu thread, continuous
    batching); its prompt tokens must attend over the paged cache like every
    later step, and a long prompt may be cut into chunks.  Reading (the pages
    give no formula): the chunk is the last n = query_start[s+1] -
    query_start[s] tokens of the sequence, so its i-th row is the token at
    position ctx - n + i, and, as in any autoregressive decoder, that token
    attends to the tokens at positions 0 .. ctx - n + i:

        out[query_start[s] + i, h] = softmax(scale * K[:p+1] q) V[:p+1],
        p = ctx - n + i,  K, V of kv-head h // (H / Hkv).

    With n = 1 this is ``decode``; ``alibi_slopes`` adds slope_h * (t - p)
    to the logit of token t as there.  n > ctx is rejected.  ``rows``
    (optional) limits the computation to those row indices of q; the other
    output rows are left NaN.  Returns out [T, H, D] float64.
    """
    T, H, D = q.shape
    if H % num_kv_heads:
        raise ValueError("H must be a multiple of num_kv_heads")
    group = H // num_kv_heads
    sc = float(np.float32(scale))
    qs = np.asarray(query_start, dtype=np.int64)
    S = len(context_lens)
    if qs.shape != (S + 1,) or qs[0] != 0 or qs[S] != T or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must rise from 0 to the number of rows")
    wanted = np.ones(T, dtype=bool) if rows is None else np.zeros(T, dtype=bool)
    if rows is not None:
        wanted[np.asarray(rows, dtype=np.int64)] = True
    out = np.full((T, H, D), np.nan if rows is not None else 0.0, dtype=np.float64)
    qf = widen(q, dtype)
    for s in range(S):
        L = int(context_lens[s])
        n = int(qs[s + 1] - qs[s])
        if n == 0 or not wanted[qs[s]:qs[s + 1]].any():
            continue
        if n > L:
            raise ValueError("more new tokens than context")
        if (L + block_size - 1) // block_size > block_tables.shape[1]:
            raise ValueError("context longer than the block table")
        K = widen(gather_pages(k_pool, block_tables[s], L, block_size), dtype)
        V = widen(gather_pages(v_pool, block_tables[s], L, block_size), dtype)
        for i in range(n):
            row = int(qs[s]) + i
            if not wanted[row]:
                continue
            visible = L - n + i + 1          # positions 0 .. L - n + i
            for h in range(H):
                kv = h // group
                x = sc * (K[kv, :visible] @ qf[row, h])
                if alibi_slopes is not None:
                    x = x + float(np.float32(alibi_slopes[h])) * (np.arange(visible) - (visible - 1))
                w = np.exp(x - x.max())
                out[row, h] = (w @ V[kv, :visible]) / w.sum()
    return out


def rope(x: np.ndarray, positions: np.ndarray, cos_sin: np.ndarray, rot_dim: int,
         neox: bool, dtype: str) -> np.ndarray:
    """Rotary position embedding of rows x [T, heads, D], in float64.

    The showapi.com article (section 4.1) names RoPE among the position
    encodings the engine serves; the pages give no formula.  Reading (the
    usual definition): the first rot_dim entries of every head are taken in
    rot_dim / 2 pairs, pair i of token t is rotated by the angle whose
    cosine and sine are cos_sin[positions[t], i] and
    cos_sin[positions[t], rot_dim / 2 + i] (a table the caller fills, e.g.
    with angle = position * base^(-2i / rot_dim)):

        (a, b) -> (a cos - b sin,  b cos + a sin)

    Pair i is entries (i, i + rot_dim / 2) when ``neox`` (split halves) and
    entries (2i, 2i + 1) otherwise (interleaved).  Entries past rot_dim are
    unchanged.  Table values are used at their float32 values.  Returns the
    rotated rows as float64.
    """
    T, nh, D = x.shape
    if rot_dim % 2 or not 0 < rot_dim <= D:
        raise ValueError("rot_dim must be even and at most head_dim")
    xf = widen(x, dtype).copy()
    half = rot_dim // 2
    cs = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)
    for t in range(T):
        pos = int(positions[t])
        if not 0 <= pos < cs.shape[0]:
            raise IndexError(f"position {pos} outside the table")
        for i in range(half):
            c, sn = cs[pos, i], cs[pos, half + i]
            ia, ib = (i, i + half) if neox else (2 * i, 2 * i + 1)
            a = xf[t, :, ia].copy()
            b = xf[t, :, ib].copy()
            xf[t, :, ia] = a * c - b * sn
            xf[t, :, ib] = b * c + a * sn
    return xf


def reshape_and_cache(k: np.ndarray, v: np.ndarray, k_pool: np.ndarray,
                      v_pool: np.ndarray, slot_mapping: np.ndarray,
                      block_size: int):
    """Write each new token's K/V rows into its pool slot; returns new pools.

    k, v [T, Hkv, D]; pools [NB, Hkv, bs, D]; slot_mapping [T] int.
    Token i goes to physical page slot // block_size, offset
    slot % block_size, for every kv-head.  Readings: a negative slot means
    "no token" and is skipped; two tokens naming one slot would leave the
    result order-dependent, so that is rejected, as is a slot outside the
    pool.  Copies are bit-for-bit (the arrays are never converted).
    """
    kp = k_pool.copy()
    vp = v_pool.copy()
    nb = kp.shape[0]
    sl = np.asarray(slot_mapping, dtype=np.int64)
    used = sl[sl >= 0]
    if len(np.unique(used)) != len(used):
        raise ValueError("duplicate slots in one cache write")
    for i in range(len(sl)):
        slot = int(sl[i])
        if slot < 0:
            continue
        page, off = divmod(slot, block_size)
        if page >= nb:
            raise IndexError(f"slot {slot} outside the pool")
        kp[page, :, off, :] = k[i]
        vp[page, :, off, :] = v[i]
    return kp, vp


def copy_blocks(k_src: np.ndarray, v_src: np.ndarray, k_dst: np.ndarray,
                v_dst: np.ndarray, block_mapping: np.ndarray):
    """Copy whole pages between pools; returns the new destination pools.

    block_mapping [N, 2] int: pair i copies page block_mapping[i, 0] of the
    source pools to page block_mapping[i, 1] of the destination pools, every
    kv-head, K and V, bit for bit.  This is the page move behind two things
    the tutorial page describes: giving a sequence its own copy of a page it
    shares with others before writing into it (section 4.2, shared pages),
    and moving a preempted sequence's pages to a CPU-side pool and back
    (sections 4.4 and 4.5).  Readings: the source and destination may be the
    same pool (pass the same arrays); two pairs naming one destination page,
    or a destination page that is also some pair's source when the pools
    are the same, would make the result order-dependent, so both are
    rejected, as is a page index outside its pool.
    """
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    same = k_src is k_dst
    kd = k_dst.copy()
    vd = v_dst.copy()
    src, dst = m[:, 0], m[:, 1]
    if len(np.unique(dst)) != len(dst):
        raise ValueError("two pairs write the same destination page")
    if same and np.intersect1d(src, dst).size:
        raise ValueError("a destination page is also a source page")
    for i in range(len(m)):
        s_page, d_page = int(src[i]), int(dst[i])
        if not (0 <= s_page < k_src.shape[0] and 0 <= d_page < kd.shape[0]):
            raise IndexError(f"pair {i} ({s_page} -> {d_page}) outside the pools")
        kd[d_page] = k_src[s_page]
        vd[d_page] = v_src[s_page]
    return kd, vd
