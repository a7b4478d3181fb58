"""reshape_and_cache on the GPU: bit-exact against the oracle's assignment,
whole pool compared as raw bits; and the write-then-attend decode step."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, compare, oracle_inputs, small_config, upload
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

BITS = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def bits(t):
    return t.detach().cpu().view(BITS[t.dtype]).numpy()


@pytest.mark.parametrize("dtype,H_kv,D,BS", [("f32", 2, 64, 16), ("bf16", 8, 128, 16),
                                              ("f16", 4, 128, 32), ("bf16", 2, 64, 32)])
def test_cache_write_bit_exact(dtype, H_kv, D, BS):
    cfg = small_config(dtype, H_kv, 1, D, BS, (40, 300, 17), extra_blocks=40)
    inp = I.generate(cfg)
    rng = np.random.default_rng(5)
    N = inp.num_blocks
    T = 300
    slots = rng.choice(N * BS, size=T, replace=False).astype(np.int64)
    slots[::17] = -1                      # padding entries
    slots[5] = N * BS + 3                 # past the pool: dropped
    key = torch.randn(T, H_kv, D).to(inp.key_cache.dtype)
    val = torch.randn(T, H_kv, D).to(inp.key_cache.dtype)
    kc, vc = inp.key_cache.to(DEV), inp.value_cache.to(DEV)
    ops.reshape_and_cache(key.to(DEV), val.to(DEV), kc, vc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    keep = slots < N * BS
    rk, rv = oracle.reshape_and_cache(bits(key)[keep], bits(val)[keep], bits(inp.key_cache),
                                      bits(inp.value_cache), slots[keep])
    assert np.array_equal(bits(kc), rk)
    assert np.array_equal(bits(vc), rv)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "int8"])
def test_slot_check_rejects_before_writing(kind, monkeypatch):
    # with the check on, a duplicate slot or one past the pool raises before
    # any launch: the caches keep their bits; with it off (the default) the
    # same distinct-slot write goes through
    N, H_kv, BS, D, T = 8, 2, 16, 64, 5
    code = {"bf16": torch.bfloat16, "fp8": torch.uint8, "int8": torch.int8}[kind]
    kc = torch.zeros(N, H_kv, BS, D, dtype=code, device=DEV)
    vc = torch.zeros_like(kc)
    key = torch.randn(T, H_kv, D, dtype=torch.bfloat16, device=DEV)
    val = torch.randn_like(key)
    write = {"bf16": lambda sm, **kw: ops.reshape_and_cache(key, val, kc, vc, sm, **kw),
             "fp8": lambda sm, **kw: ops.reshape_and_cache_fp8(key, val, kc, vc, sm, 0.05, 0.05, **kw),
             "int8": lambda sm, **kw: ops.reshape_and_cache_i8(key, val, kc, vc, sm, 0.05, 0.05, **kw)}[kind]
    dup = torch.tensor([3, 40, -1, 9, 40], dtype=torch.int64, device=DEV)
    past = torch.tensor([3, 4, N * BS, 9, 10], dtype=torch.int64, device=DEV)
    with pytest.raises(RuntimeError, match="slot 40 given to tokens 1 and 4"):
        write(dup, check_slots=True)
    monkeypatch.setenv("PAGEDATTN_CHECK_SLOTS", "1")
    with pytest.raises(RuntimeError, match="past the pool"):
        write(past)
    torch.cuda.synchronize()
    assert not kc.view(torch.uint8).any() and not vc.view(torch.uint8).any()
    monkeypatch.delenv("PAGEDATTN_CHECK_SLOTS")
    write(torch.tensor([3, 40, -1, 9, 41], dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert kc.view(torch.uint8)[40 // BS, :, 40 % BS].any()


def test_write_then_attend_tiny():
    """The append flow: each sequence's next token goes to position L_b (a
    free block when L_b is a multiple of the block size), then decode attends
    over L_b + 1 tokens."""
    cfg = I.CONFIGS["tiny_fp32"]
    inp = I.generate(cfg)
    BS = cfg.block_size
    L = inp.context_lens.numpy().copy()
    bt = inp.block_tables.numpy().copy()
    free = list(inp.free_blocks)
    slots = []
    for b in range(cfg.num_seqs):
        pos = int(L[b])
        if pos % BS == 0:
            bt[b, pos // BS] = free.pop(0)
        slots.append(int(bt[b, pos // BS]) * BS + pos % BS)
    slots = np.array(slots, dtype=np.int64)
    key = inp.new_key[:cfg.num_seqs]
    val = inp.new_value[:cfg.num_seqs]
    d = upload(inp)
    ops.reshape_and_cache(key.to(DEV), val.to(DEV), d["key_cache"], d["value_cache"],
                          torch.from_numpy(slots).to(DEV))
    bt_t = torch.from_numpy(bt.astype(np.int32)).to(DEV)
    lens_t = torch.from_numpy((L + 1).astype(np.int32)).to(DEV)
    out = ops.paged_attention_decode(d["query"], d["key_cache"], d["value_cache"], bt_t, lens_t)
    torch.cuda.synchronize()
    kc, vc = oracle.reshape_and_cache(key.numpy(), val.numpy(), inp.key_cache.numpy(),
                                      inp.value_cache.numpy(), slots)
    assert np.array_equal(d["key_cache"].cpu().numpy(), kc)
    ref = oracle.decode_contiguous(inp.query.numpy(), kc, vc, bt, L + 1, cfg.scale)
    compare(out, ref, "f32", what="write then attend")


def test_tiny_config_cache_write():
    inp = I.generate(I.CONFIGS["tiny_fp32"])
    d = upload(inp)
    ops.reshape_and_cache(d["new_key"], d["new_value"], d["key_cache"], d["value_cache"],
                          d["slot_mapping"])
    torch.cuda.synchronize()
    rk, rv = oracle.reshape_and_cache(bits(inp.new_key), bits(inp.new_value),
                                      bits(inp.key_cache), bits(inp.value_cache),
                                      inp.slot_mapping.numpy())
    assert np.array_equal(bits(d["key_cache"]), rk)
    assert np.array_equal(bits(d["value_cache"]), rv)


@pytest.mark.parametrize("name,kernel,partition_size", [
    ("qwen7b_gqa_bf16", ops.KERNEL_AUTO, 0),       # matrix core, balanced schedule
    ("qwen7b_gqa_bf16", ops.KERNEL_MFMA, 256),     # matrix core, fixed partitions
    ("qwen7b_gqa_bf16", ops.KERNEL_GENERIC, 0),    # vector ALU: append kernel + decode
    ("long_ctx_bf16", ops.KERNEL_AUTO, 0),
    ("tiny_fp32", ops.KERNEL_AUTO, 0),
    ("qwen7b_gqa_bf16:mqa64", ops.KERNEL_AUTO, 0),   # 64 heads on 1 KV head: two passes
    ("qwen7b_gqa_bf16:mqa64", ops.KERNEL_MFMA, 256),
    ("qwen7b_gqa_bf16:g37", ops.KERNEL_AUTO, 0),     # 37 heads per KV head: 19 + 18
])
def test_decode_append_equals_write_then_decode(name, kernel, partition_size):
    """The fused step gives bit for bit the caches and output of
    reshape_and_cache at each sequence's last position followed by decode."""
    base, _, variant = name.partition(":")
    cfg = I.CONFIGS[base]
    if variant == "mqa64":
        cfg = I.with_overrides(cfg, num_seqs=16, num_heads=64, num_kv_heads=1)
    elif variant == "g37":
        cfg = I.with_overrides(cfg, num_seqs=16, num_heads=74, num_kv_heads=2)
    inp = I.generate(cfg, new_tokens_at="last")
    prev = ops.select_kernel(kernel)
    try:
        d1 = upload(inp)
        ops.reshape_and_cache(d1["new_key"], d1["new_value"], d1["key_cache"],
                              d1["value_cache"], d1["slot_mapping"])
        o1 = ops.paged_attention_decode(d1["query"], d1["key_cache"], d1["value_cache"],
                                        d1["block_tables"], d1["context_lens"],
                                        partition_size=partition_size)
        d2 = upload(inp)
        o2 = ops.decode_append(d2["query"], d2["new_key"], d2["new_value"], d2["key_cache"],
                               d2["value_cache"], d2["block_tables"], d2["context_lens"],
                               partition_size=partition_size)
        torch.cuda.synchronize()
    finally:
        ops.select_kernel(prev)
    assert torch.equal(o1, o2)
    assert torch.equal(d1["key_cache"], d2["key_cache"])
    assert torch.equal(d1["value_cache"], d2["value_cache"])


@pytest.mark.parametrize("head_dim", [64, 256])
@pytest.mark.parametrize("partition_size", [0, 256])
def test_decode_append_other_head_dims_equals_write_then_decode(partition_size, head_dim):
    """The matrix-core kernel's own append step at head_dim 64 and 256 (8 and
    32 lanes per row) against reshape_and_cache followed by decode, bit for
    bit."""
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=12, num_blocks=4000,
                           head_dim=head_dim)
    inp = I.generate(cfg, new_tokens_at="last")
    d1 = upload(inp)
    ops.reshape_and_cache(d1["new_key"], d1["new_value"], d1["key_cache"], d1["value_cache"],
                          d1["slot_mapping"])
    o1 = ops.paged_attention_decode(d1["query"], d1["key_cache"], d1["value_cache"],
                                    d1["block_tables"], d1["context_lens"],
                                    partition_size=partition_size)
    d2 = upload(inp)
    o2 = ops.decode_append(d2["query"], d2["new_key"], d2["new_value"], d2["key_cache"],
                           d2["value_cache"], d2["block_tables"], d2["context_lens"],
                           partition_size=partition_size)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(d1["key_cache"], d2["key_cache"])
    assert torch.equal(d1["value_cache"], d2["value_cache"])


def test_decode_append_against_oracle():
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=6, num_blocks=400,
                           max_blocks_per_seq=64, lens_kind="list",
                           lens_args=(1, 16, 17, 33, 500, 1024))
    inp = I.poison_unread(I.generate(cfg, new_tokens_at="last"))
    d = upload(inp)
    out = ops.decode_append(d["query"], d["new_key"], d["new_value"], d["key_cache"],
                            d["value_cache"], d["block_tables"], d["context_lens"])
    torch.cuda.synchronize()
    kc, vc = oracle.reshape_and_cache(bits(inp.new_key), bits(inp.new_value),
                                      bits(inp.key_cache), bits(inp.value_cache),
                                      inp.slot_mapping.numpy())
    assert np.array_equal(bits(d["key_cache"]), kc)
    assert np.array_equal(bits(d["value_cache"]), vc)
    kcf = torch.from_numpy(kc).view(torch.bfloat16).float().numpy()
    vcf = torch.from_numpy(vc).view(torch.bfloat16).float().numpy()
    ref = oracle.decode_contiguous(inp.query.float().numpy(), kcf, vcf,
                                   inp.block_tables.numpy(), inp.context_lens.numpy(), cfg.scale)
    compare(out, ref, "bf16", what="decode_append vs oracle")
