"""Seeded input generators (CPU only): determinism and table structure."""

import numpy as np
import torch

from paged_kv_decode_attention_amd import inputs as I


def test_deterministic_and_seed_sensitive():
    cfg = I.CONFIGS["tiny_fp32"]
    a, b = I.generate(cfg), I.generate(cfg)
    for f in ("query", "key_cache", "value_cache", "block_tables", "context_lens",
              "new_key", "new_value", "slot_mapping"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    c = I.generate(cfg, seed=99)
    assert not torch.equal(a.query, c.query)


def test_tiny_tables_no_reuse_and_free_slots():
    inp = I.generate(I.CONFIGS["tiny_fp32"])
    bt = inp.block_tables.numpy()
    L = inp.context_lens.numpy()
    assert L.min() >= 1 and L.max() <= 64
    used = []
    for b in range(bt.shape[0]):
        n = -(-int(L[b]) // 16)
        assert (bt[b, :n] >= 0).all() and (bt[b, n:] == -1).all()
        used += bt[b, :n].tolist()
    assert len(used) == len(set(used))
    slots = inp.slot_mapping.numpy()
    assert len(set(slots.tolist())) == len(slots) == 4
    assert set((slots // 16).tolist()) <= set(inp.free_blocks.tolist())
    assert not set((slots // 16).tolist()) & set(used)


def test_shared_prefix_structure():
    cfg = I.CONFIGS["mixed_shared_bf16"]
    # small pool draw is enough to check the table layout: shrink the heads
    cfg = I.with_overrides(cfg, num_heads=8, num_kv_heads=2, head_dim=16)
    inp = I.generate(cfg)
    bt = inp.block_tables.numpy()
    L = inp.context_lens.numpy()
    assert L.min() >= 1 and L.max() <= 8192
    shared = inp.extras["shared_blocks"]
    owner = {}
    for b in range(128):
        g = b // 32
        n = -(-int(L[b]) // 16)
        k = min(n, 64)
        assert (bt[b, :k] == shared[g][:k]).all()
        for blk in bt[b, k:n].tolist():      # private tails are not shared
            assert blk not in owner
            owner[blk] = b
    assert not set(owner) & set(shared.ravel().tolist())


def test_poison_marks_only_unread_slots():
    inp = I.generate(I.CONFIGS["tiny_fp32"])
    clean = inp.key_cache.clone()
    I.poison_unread(inp)
    bt = inp.block_tables.numpy()
    for b, L in enumerate(inp.context_lens.numpy().tolist()):
        for pos in range(L):
            blk = bt[b, pos // 16]
            assert torch.equal(inp.key_cache[blk, :, pos % 16], clean[blk, :, pos % 16])
    assert torch.isnan(inp.key_cache).any()


def test_last_slot_mode_points_at_final_position():
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_blocks=4096,
                           lens_kind="uniform", lens_args=(1, 200))
    inp = I.generate(cfg, new_tokens_at="last")
    bt = inp.block_tables.numpy()
    for b, L in enumerate(inp.context_lens.numpy().tolist()):
        s = int(inp.slot_mapping[b])
        assert s // 16 == bt[b, (L - 1) // 16] and s % 16 == (L - 1) % 16
