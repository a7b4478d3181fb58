"""INT8 KV cache on the GPU: the quantised cache write bit-exact against the
oracle over every bf16 bit pattern, decode over INT8 caches against the
float64 oracle on the dequantised caches, and the fused append equal to the
write followed by the decode."""

import numpy as np
import pytest
import torch

import oracle
from oracle import int8
from gpu_util import DEV, compare, small_config
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

# unit-variance data: +-127 codes span about +-5.3 (keys) and +-6.4 (values),
# so the largest draws saturate
K_SCALE, V_SCALE = 1.0 / 24, 1.0 / 20
RAGGED = (1, 15, 16, 17, 31, 33, 100, 513)
POISON = 1.0e4        # unread slots: saturates to code 127, which a read would show


def quantize_pool(cache, scale, chunk=1 << 24):
    """Oracle INT8 codes (uint8 bytes) of a (bf16/f16) pool, in pieces."""
    x = cache.float().numpy().reshape(-1)
    out = np.empty(x.shape, dtype=np.uint8)
    for i in range(0, x.size, chunk):
        out[i:i + chunk] = int8.quantize(x[i:i + chunk], scale)
    return out.reshape(cache.shape)


def i8_inputs(inp):
    kq = quantize_pool(inp.key_cache, K_SCALE)
    vq = quantize_pool(inp.value_cache, V_SCALE)
    return kq, vq, int8.dequantize(kq, K_SCALE), int8.dequantize(vq, V_SCALE)


def dev_codes(codes):
    return torch.from_numpy(codes.view(np.int8)).to(DEV)


def oracle_i8(inp, kdq, vdq, pairs=None):
    return oracle.decode_contiguous(inp.query.float().numpy(), kdq, vdq,
                                    inp.block_tables.numpy().astype(np.int64),
                                    inp.context_lens.numpy().astype(np.int64), inp.cfg.scale,
                                    pairs=pairs)


def run_i8(inp, kq, vq, partition_size=0, **kw):
    out = ops.paged_attention_decode_i8(
        inp.query.to(DEV), dev_codes(kq), dev_codes(vq), inp.block_tables.to(DEV),
        inp.context_lens.to(DEV), K_SCALE, V_SCALE, partition_size=partition_size, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("src", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (K_SCALE, V_SCALE), (3.0, 0.37)])
def test_i8_cache_write_bit_exact(src, scales):
    T, H_kv, D, BS, N = 256, 2, 128, 16, 64
    if src == torch.bfloat16:
        # every bf16 bit pattern, NaN and infinities included, as keys; the
        # values the same patterns reversed
        pat = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
        key = pat.view(torch.bfloat16).reshape(T, H_kv, D)
        value = key.flip(0)
    else:
        # spread so that ties (x.5 after scaling), saturation and small codes
        # all occur
        g = torch.Generator().manual_seed(9)
        key = (torch.randn(T, H_kv, D, generator=g) * 40).to(src)
        value = torch.round(torch.randn(T, H_kv, D, generator=g) * 200).to(src) / 2
    rng = np.random.default_rng(4)
    slots = rng.choice(N * BS, size=T, replace=False).astype(np.int64)
    slots[::31] = -1
    kc = torch.full((N, H_kv, BS, D), 0x55, dtype=torch.int8)
    vc = kc.clone()
    dk, dv = kc.to(DEV), vc.to(DEV)
    ops.reshape_and_cache_i8(key.to(DEV), value.to(DEV), dk, dv, torch.from_numpy(slots).to(DEV),
                             *scales)
    torch.cuda.synchronize()
    rk, rv = int8.reshape_and_cache_i8(key.float().numpy(), value.float().numpy(),
                                       kc.numpy().view(np.uint8), vc.numpy().view(np.uint8),
                                       slots, *scales)
    assert np.array_equal(dk.cpu().numpy().view(np.uint8), rk)
    assert np.array_equal(dv.cpu().numpy().view(np.uint8), rv)


CASES = [("bf16", 2, 7, 128, 16), ("bf16", 2, 4, 128, 32), ("f16", 2, 4, 128, 16),
         ("bf16", 1, 16, 128, 16), ("f16", 3, 1, 128, 32), ("bf16", 2, 7, 128, 64),
         ("bf16", 2, 7, 64, 16), ("f16", 2, 4, 64, 32), ("bf16", 1, 16, 64, 64),
         ("bf16", 2, 7, 256, 16), ("f16", 1, 8, 256, 32), ("bf16", 2, 7, 128, 8),
         ("f16", 2, 4, 64, 8), ("bf16", 1, 32, 128, 16), ("f16", 2, 20, 64, 32),
         # groups split into passes: 2 x 32 heads, 2 x 16 at head_dim 256,
         # uneven: 19 + 18 heads, and 13 + 13 + 11 at head_dim 256
         ("bf16", 1, 64, 128, 16), ("f16", 1, 32, 256, 16), ("bf16", 1, 37, 128, 16),
         ("f16", 1, 37, 256, 32)]


@pytest.mark.parametrize("partition_size", [0, 64, 256])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-hkv%d-g%d-d%d-bs%d" % c)
def test_i8_decode_parity(case, partition_size):
    dtype, H_kv, G, D, BS = case
    if partition_size % BS:
        pytest.skip("partition not a multiple of the block size")
    inp = I.poison_unread(I.generate(small_config(dtype, H_kv, G, D, BS, RAGGED)), POISON)
    kq, vq, kdq, vdq = i8_inputs(inp)
    out = run_i8(inp, kq, vq, partition_size)
    compare(out, oracle_i8(inp, kdq, vdq), dtype, what="int8 %s P=%d" % (case, partition_size))


def test_i8_code_minus_128_and_errors():
    """A stored -128 (never written by the encoder) reads as -128; bad scales,
    cache dtypes and the generic kernel are refused."""
    inp = I.generate(small_config("bf16", 2, 7, 128, 16, (40, 70)))
    kq, vq, _, _ = i8_inputs(inp)
    rng = np.random.default_rng(11)
    for c in (kq, vq):
        c.reshape(-1)[rng.choice(c.size, size=c.size // 50, replace=False)] = 0x80
    out = run_i8(inp, kq, vq)
    compare(out, oracle_i8(inp, int8.dequantize(kq, K_SCALE), int8.dequantize(vq, V_SCALE)),
            "bf16", what="codes -128")
    with pytest.raises(RuntimeError, match="finite and positive"):
        ops.paged_attention_decode_i8(
            inp.query.to(DEV), dev_codes(kq), dev_codes(vq), inp.block_tables.to(DEV),
            inp.context_lens.to(DEV), K_SCALE, float("inf"))
    with pytest.raises(ValueError, match="int8"):
        ops.paged_attention_decode_i8(
            inp.query.to(DEV), torch.from_numpy(kq).to(DEV), torch.from_numpy(vq).to(DEV),
            inp.block_tables.to(DEV), inp.context_lens.to(DEV), K_SCALE, V_SCALE)
    prev = ops.select_kernel(ops.KERNEL_GENERIC)
    try:
        with pytest.raises(RuntimeError, match="matrix-core"):
            run_i8(inp, kq, vq)
    finally:
        ops.select_kernel(prev)


@pytest.mark.parametrize("head_dim", [128, 64, 256])
@pytest.mark.parametrize("partition_size", [0, 256])
def test_i8_decode_append_equals_write_then_decode(partition_size, head_dim):
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=12, num_blocks=4000,
                           head_dim=head_dim)
    inp = I.generate(cfg, new_tokens_at="last")
    kq, vq, _, _ = i8_inputs(inp)
    q = inp.query.to(DEV)
    nk, nv = inp.new_key.to(DEV), inp.new_value.to(DEV)
    bt, cl = inp.block_tables.to(DEV), inp.context_lens.to(DEV)
    k1, v1 = dev_codes(kq), dev_codes(vq)
    k2, v2 = k1.clone(), v1.clone()
    ops.reshape_and_cache_i8(nk, nv, k1, v1, inp.slot_mapping.to(DEV), K_SCALE, V_SCALE)
    o1 = ops.paged_attention_decode_i8(q, k1, v1, bt, cl, K_SCALE, V_SCALE,
                                       partition_size=partition_size)
    o2 = ops.decode_append_i8(q, nk, nv, k2, v2, bt, cl, K_SCALE, V_SCALE,
                              partition_size=partition_size)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(o1, o2)
    # and against the oracle: the appended rows quantised by the oracle
    rk, rv = int8.reshape_and_cache_i8(inp.new_key.float().numpy(),
                                       inp.new_value.float().numpy(), kq, vq,
                                       inp.slot_mapping.numpy(), K_SCALE, V_SCALE)
    assert np.array_equal(k1.cpu().numpy().view(np.uint8), rk)
    assert np.array_equal(v1.cpu().numpy().view(np.uint8), rv)
    ref = oracle_i8(inp, int8.dequantize(rk, K_SCALE), int8.dequantize(rv, V_SCALE))
    compare(o2, ref, "bf16", what="int8 decode_append")


def test_i8_full_bench_workload_sampled():
    """The Qwen-shaped bench workload (64 sequences, 20000-block pool) on INT8
    caches, checked on sampled (sequence, head) pairs."""
    inp = I.generate(I.CONFIGS["qwen7b_gqa_bf16"])
    kq, vq, _, _ = i8_inputs(inp)
    out = run_i8(inp, kq, vq)
    rng = np.random.default_rng(5)
    pairs = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 64, 48),
                                                      rng.integers(0, 28, 48))})
    used = sorted({b for b, _ in pairs})
    blocks = np.unique(np.concatenate([inp.block_tables[b].numpy() for b in used]))
    blocks = blocks[blocks >= 0]
    kdq = np.zeros(kq.shape, dtype=np.float64)
    vdq = np.zeros(vq.shape, dtype=np.float64)
    kdq[blocks] = int8.dequantize(kq[blocks], K_SCALE)
    vdq[blocks] = int8.dequantize(vq[blocks], V_SCALE)
    compare(out, oracle_i8(inp, kdq, vdq, pairs), "bf16", pairs=pairs, what="int8 bench workload")


@pytest.mark.parametrize("D", [48, 256])
def test_i8_cache_write_other_head_dims(D):
    """head_dim 48 (a multiple of 16 that is not a power of two) and 256."""
    T, H_kv, BS, N = 100, 3, 32, 16
    g = torch.Generator().manual_seed(D)
    key = (torch.randn(T, H_kv, D, generator=g) * 3).to(torch.bfloat16)
    value = (torch.randn(T, H_kv, D, generator=g) * 9).to(torch.float16)
    slots = np.random.default_rng(D).choice(N * BS, size=T, replace=False).astype(np.int64)
    kc = torch.full((N, H_kv, BS, D), -3, dtype=torch.int8)
    dk, dv = kc.to(DEV), kc.to(DEV)
    ops.reshape_and_cache_i8(key.to(DEV), value.to(torch.bfloat16).to(DEV), dk, dv,
                             torch.from_numpy(slots).to(DEV), K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    rk, rv = int8.reshape_and_cache_i8(key.float().numpy(),
                                       value.to(torch.bfloat16).float().numpy(),
                                       kc.numpy().view(np.uint8), kc.numpy().view(np.uint8),
                                       slots, K_SCALE, V_SCALE)
    assert np.array_equal(dk.cpu().numpy().view(np.uint8), rk)
    assert np.array_equal(dv.cpu().numpy().view(np.uint8), rv)
