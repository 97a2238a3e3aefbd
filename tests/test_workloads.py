"""CPU checks of the seeded input generator (structure, not arithmetic)."""
import math

import numpy as np
import pytest
import torch

from paged_kv_cache_457_amd.workloads import (build_workload, make_config,
                                              round_f32_to_bf16_bits)


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8], np.float32)])
    ours = round_f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def _check_structure(w):
    bs = w.block_size
    S = w.num_seqs
    owners = {}
    for s in range(S):
        L = int(w.context_lens[s])
        n = (L + bs - 1) // bs
        row = w.block_tables[s]
        assert np.all((row[:n] >= 0) & (row[:n] < w.num_blocks))
        assert np.all(row[n:] == -1)
        for j in range(n):
            owners.setdefault(int(row[j]), set()).add(s)
        # the append slot is position ctx-1
        if L:
            pos = L - 1
            assert w.slot_mapping[s] == row[pos // bs] * bs + pos % bs
    for page, who in owners.items():
        assert w.refcount[page] == len(who)
    used = w.slot_mapping[w.slot_mapping >= 0]
    assert len(np.unique(used)) == len(used)
    # poison: the append slots hold NaN before the append
    for sl in used:
        p, o = divmod(int(sl), bs)
        vals = w.k_pool[p, :, o, :]
        if w.dtype == "f32":
            assert np.all(np.isnan(vals))
        else:
            assert np.all(vals == 0x7FC0)


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_configs_match_their_descriptions(idx):
    w = make_config(idx)
    _check_structure(w)
    assert w.scale == np.float32(1.0 / math.sqrt(w.head_dim))
    if idx == 1:
        assert list(w.context_lens) == [1, 17, 33, 100]
        assert (w.num_heads, w.num_kv_heads, w.head_dim, w.block_size, w.dtype) == (4, 4, 64, 16, "f32")
        assert w.num_blocks == 64
        fs = w.extra["free_slots"]
        assert len(np.unique(fs)) == 4
        live = w.extra["live"]
        for sl in fs:
            assert not live[sl // 16, sl % 16]
            assert sl not in set(w.slot_mapping.tolist())
    elif idx == 2:
        assert w.num_seqs == 64 and (w.num_heads, w.num_kv_heads, w.head_dim) == (32, 32, 128)
        assert w.context_lens.min() >= 128 and w.context_lens.max() <= 2048
        needed = int(((w.context_lens + 15) // 16).sum())
        assert w.num_blocks == math.ceil(1.25 * needed)
        assert w.max_blocks_per_seq == 128
    elif idx == 3:
        assert w.num_seqs == 256 and (w.num_heads, w.num_kv_heads) == (32, 8)
        assert w.context_lens.min() >= 16 and w.context_lens.max() <= 8192
        assert 300 < np.median(w.context_lens) < 800
    elif idx == 4:
        assert w.num_seqs == 8 and np.all(w.context_lens == 32768) and w.block_size == 32
        assert w.max_blocks_per_seq == 1024
    elif idx == 5:
        assert w.num_seqs == 128
        div = w.extra["divergent"]
        assert np.all(w.context_lens == 1024 + div + 1)
        assert np.all((div >= 0) & (div <= 256))
        # sample 0 of every prompt appends on a fresh page
        assert np.all(div.reshape(16, 8)[:, 0] % 16 == 0)
        for p in range(16):
            rows = w.block_tables[p * 8:(p + 1) * 8, :64]
            assert np.all(rows == rows[0])                  # shared prefix pages
            assert np.all(w.refcount[rows[0]] == 8)
        assert np.all(w.refcount[w.slot_mapping // 16] == 1)


def test_determinism():
    a = build_workload("a", [3, 40], 4, 2, 16, 16, "bf16", seed=5)
    b = build_workload("b", [3, 40], 4, 2, 16, 16, "bf16", seed=5)
    for name in ("q", "k_pool", "v_pool", "block_tables", "k_new", "v_new", "slot_mapping"):
        assert np.array_equal(getattr(a, name), getattr(b, name))


def test_ctx_zero_has_no_pages_and_no_slot():
    w = build_workload("z", [0, 5], 2, 2, 8, 4, "f32", seed=1)
    assert np.all(w.block_tables[0] == -1) and w.slot_mapping[0] == -1
