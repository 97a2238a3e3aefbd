"""Per-element error bound of a bf16 decode result against the fp64 oracle.

The library computes in fp32 and rounds the result to bf16 (nearest even).
For an output element with exact value r, fp32 value o before rounding and
bf16 result g:

    |g - r| <= |g - o| + |o - r| <= ulp(|o|) / 2 + delta <= ulp(|r|) + delta,

since ulp(|o|) <= 2 ulp(|r|) when |o - r| is small against |r| (at most one
binade up).  ``delta`` bounds the fp32 error |o - r|.  With M_V the largest
|V| of any live token, u the unit roundoff of one fp32 operation and
o = sum_t p_t V_t / sum_t p_t, p_t = exp(l_t - m):

* weights as a bf16 pair (matrix-core P.V): p = hi + lo + e with
  |e| <= 2^-18 p (hi = bf16(p), lo = bf16(p - hi), each with 8 significant
  bits), so the weighted sum moves by at most 2^-18 M_V;
* accumulation: each term p_t V_t (and p_t) passes through at most k
  roundings (sequential adds within a partition's wave, rescales by
  exp(m_old - m_new), the merge of waves and of partitions, the final
  division), so numerator and denominator are each off by at most k u of
  their sum of magnitudes: 2 k u M_V;
* logits: l_t = scale * q . K_t summed in fp32 over D exact bf16 products
  is off by at most scale * D * u * A, A = max_t sum_d |q_d K_td|; the
  log2(e) fold, the subtraction of the max and the exp2 add about
  u * (2 scale A + 2) more.  A uniform logit error E changes o by at most
  E * max_t |V_t - o| <= 2 M_V E.

k is bounded from the partition length: within a partition a lane adds at
most one term per 4 tokens (one query head per kv-head, on the VALU) or
one per 16-token granule plus the 16 sums inside a matrix instruction, and
rescales at most once per page or granule; then at most 8 waves and P
partitions are merged: k <= part_tokens / 8 + P + 32.

u is 2^-24 (round to nearest) for the VALU paths.  The matrix cores'
rounding of their internal sums is not documented, so where they take
part u is 2^-23 (one full ulp per addition).

This is a worst-case bound: it holds for every summation order, so it does
not depend on how the kernels order their sums.
"""
from __future__ import annotations

import numpy as np

import oracle

U_NEAREST = 2.0 ** -24
U_MATRIX = 2.0 ** -23


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits); the smallest
    normal spacing below the normal range."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def max_abs_dot(q_bits, kp_bits, block_tables, context_lens, num_kv_heads, block_size,
                dtype) -> float:
    """A = max over sequences, query heads and live tokens of
    sum_d |q_d| |K_td| (tokens gathered through the table)."""
    S, H, D = q_bits.shape
    G = H // num_kv_heads
    best = 0.0
    for s in range(S):
        L = int(context_lens[s])
        if L <= 0:
            continue
        k = oracle.gather_pages(kp_bits, block_tables[s], L, block_size)   # [Hkv, L, D]
        qa = np.abs(oracle.widen(q_bits[s], dtype)).astype(np.float32)      # [H, D]
        for g in range(num_kv_heads):
            ka = np.abs(oracle.widen(k[g], dtype)).astype(np.float32)       # [L, D]
            best = max(best, float((ka @ qa[g * G:(g + 1) * G].T).max()))
    return best * (1 + 1e-5)      # the float32 product above is itself rounded


def max_abs_live(pool_bits, dtype) -> float:
    """M_V: the largest |V| in the pool, dead (NaN-poisoned) slots ignored.
    bf16 magnitudes order like their bit patterns with the sign cleared, so
    the largest finite pattern is found on the raw bits."""
    if dtype == "bf16":
        mag = np.asarray(pool_bits, dtype=np.uint16).reshape(-1) & np.uint16(0x7FFF)
        finite = mag[mag < np.uint16(0x7F80)]
        return float(oracle.widen(finite.max(initial=np.uint16(0)), "bf16"))
    return float(np.nanmax(np.abs(np.asarray(pool_bits, dtype=np.float32))))


def fp32_delta(*, m_v: float, a_dot: float, scale: float, head_dim: int, part_tokens: int,
               parts: int, matrix_cores: bool) -> float:
    """delta of the module docstring for one call's shapes and data."""
    u = U_MATRIX if matrix_cores else U_NEAREST
    k = part_tokens / 8 + parts + 32
    pair = 2.0 ** -18 * m_v if matrix_cores else 0.0
    accumulate = 2 * k * u * m_v
    logit = u * (scale * head_dim * a_dot + 2 * scale * a_dot + 2)
    return pair + accumulate + 2 * m_v * logit


def check_ulp_bound(got_bits, ref, delta: float):
    """Max of |g - r| / (ulp(|r|) + delta) over all elements (must be <= 1)
    and the element where it peaks."""
    g = oracle.widen(got_bits, "bf16")
    ratio = np.abs(g - ref) / (bf16_ulp(ref) + delta)
    i = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    return (float(ratio[i]) if ratio.size else 0.0), i
