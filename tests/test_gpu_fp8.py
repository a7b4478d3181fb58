"""FP8 (OCP E4M3) KV cache on the GPU: the quantised cache write bit-exact
against the oracle over every bf16 bit pattern, and decode over E4M3 caches
against the float64 oracle on the dequantised caches."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from gpu_util import DEV, compare, small_config
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 1.0 / 64, 1.0 / 48
RAGGED = (1, 15, 16, 17, 31, 33, 100, 513)


def quantize_pool(cache, scale, chunk=1 << 24):
    """Oracle E4M3 codes of a (bf16/f16) pool, in pieces to bound memory."""
    x = cache.float().numpy().reshape(-1)
    out = np.empty(x.shape, dtype=np.uint8)
    for i in range(0, x.size, chunk):
        out[i:i + chunk] = fp8.quantize(x[i:i + chunk], scale)
    return out.reshape(cache.shape)


def fp8_inputs(inp):
    """E4M3 caches of a generated workload (unread slots hold NaN codes when
    the workload was poisoned) and the oracle's dequantised caches."""
    kq = quantize_pool(inp.key_cache, K_SCALE)
    vq = quantize_pool(inp.value_cache, V_SCALE)
    return kq, vq, fp8.dequantize(kq, K_SCALE), fp8.dequantize(vq, V_SCALE)


def oracle_fp8(inp, kdq, vdq, pairs=None):
    return oracle.decode_contiguous(inp.query.float().numpy(), kdq, vdq,
                                    inp.block_tables.numpy().astype(np.int64),
                                    inp.context_lens.numpy().astype(np.int64), inp.cfg.scale,
                                    pairs=pairs)


def run_fp8(inp, kq, vq, partition_size=0, **kw):
    out = ops.paged_attention_decode_fp8(
        inp.query.to(DEV), torch.from_numpy(kq).to(DEV), torch.from_numpy(vq).to(DEV),
        inp.block_tables.to(DEV), inp.context_lens.to(DEV), K_SCALE, V_SCALE,
        partition_size=partition_size, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("src", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("scales", [(1.0, 1.0), (K_SCALE, V_SCALE), (3.0, 0.37)])
def test_fp8_cache_write_bit_exact(src, scales):
    T, H_kv, D, BS, N = 256, 2, 128, 16, 64
    if src == torch.bfloat16:
        # every bf16 bit pattern, NaN and infinities included, as keys; the
        # values the same patterns reversed
        pat = torch.arange(1 << 16, dtype=torch.int32).to(torch.int16)
        key = pat.view(torch.bfloat16).reshape(T, H_kv, D)
        value = key.flip(0)
    else:
        g = torch.Generator().manual_seed(9)
        key = (torch.randn(T, H_kv, D, generator=g) * 40).to(src)
        value = (torch.randn(T, H_kv, D, generator=g) * 0.01).to(src)
    rng = np.random.default_rng(4)
    slots = rng.choice(N * BS, size=T, replace=False).astype(np.int64)
    slots[::31] = -1
    kc = torch.full((N, H_kv, BS, D), 0x55, dtype=torch.uint8)
    vc = kc.clone()
    dk, dv = kc.to(DEV), vc.to(DEV)
    ops.reshape_and_cache_fp8(key.to(DEV), value.to(DEV), dk, dv, torch.from_numpy(slots).to(DEV),
                              *scales)
    torch.cuda.synchronize()
    rk, rv = fp8.reshape_and_cache_fp8(key.float().numpy(), value.float().numpy(), kc.numpy(),
                                       vc.numpy(), slots, *scales)
    assert np.array_equal(dk.cpu().numpy(), rk)
    assert np.array_equal(dv.cpu().numpy(), rv)


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
def test_fp8_decode_parity(case, partition_size):
    dtype, H_kv, G, D, BS = case
    if partition_size % BS:
        pytest.skip("partition not a multiple of the block size")
    inp = I.poison_unread(I.generate(small_config(dtype, H_kv, G, D, BS, RAGGED)))
    kq, vq, kdq, vdq = fp8_inputs(inp)
    out = run_fp8(inp, kq, vq, partition_size)
    compare(out, oracle_fp8(inp, kdq, vdq), dtype, what="fp8 %s P=%d" % (case, partition_size))


def test_fp8_float8_tensor_type_and_errors():
    inp = I.generate(small_config("bf16", 2, 7, 128, 16, (40, 70)))
    kq, vq, kdq, vdq = fp8_inputs(inp)
    out = ops.paged_attention_decode_fp8(
        inp.query.to(DEV), torch.from_numpy(kq).to(DEV).view(torch.float8_e4m3fn),
        torch.from_numpy(vq).to(DEV).view(torch.float8_e4m3fn), inp.block_tables.to(DEV),
        inp.context_lens.to(DEV), K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    compare(out, oracle_fp8(inp, kdq, vdq), "bf16", what="float8_e4m3fn tensors")
    with pytest.raises(RuntimeError, match="finite and positive"):
        ops.paged_attention_decode_fp8(
            inp.query.to(DEV), torch.from_numpy(kq).to(DEV), torch.from_numpy(vq).to(DEV),
            inp.block_tables.to(DEV), inp.context_lens.to(DEV), 0.0, V_SCALE)
    prev = ops.select_kernel(ops.KERNEL_GENERIC)
    try:
        with pytest.raises(RuntimeError, match="matrix-core"):
            run_fp8(inp, kq, vq)
    finally:
        ops.select_kernel(prev)


@pytest.mark.parametrize("head_dim", [128, 64, 256])
@pytest.mark.parametrize("partition_size", [0, 256])
def test_fp8_decode_append_equals_write_then_decode(partition_size, head_dim):
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=12, num_blocks=4000,
                           head_dim=head_dim)
    inp = I.generate(cfg, new_tokens_at="last")
    kq, vq, _, _ = fp8_inputs(inp)
    q = inp.query.to(DEV)
    nk, nv = inp.new_key.to(DEV), inp.new_value.to(DEV)
    bt, cl = inp.block_tables.to(DEV), inp.context_lens.to(DEV)
    k1, v1 = torch.from_numpy(kq).to(DEV), torch.from_numpy(vq).to(DEV)
    k2, v2 = k1.clone(), v1.clone()
    ops.reshape_and_cache_fp8(nk, nv, k1, v1, inp.slot_mapping.to(DEV), K_SCALE, V_SCALE)
    o1 = ops.paged_attention_decode_fp8(q, k1, v1, bt, cl, K_SCALE, V_SCALE,
                                        partition_size=partition_size)
    o2 = ops.decode_append_fp8(q, nk, nv, k2, v2, bt, cl, K_SCALE, V_SCALE,
                               partition_size=partition_size)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(o1, o2)
    # and against the oracle: the appended rows quantised by the oracle
    rk, rv = fp8.reshape_and_cache_fp8(inp.new_key.float().numpy(), inp.new_value.float().numpy(),
                                       kq, vq, inp.slot_mapping.numpy(), K_SCALE, V_SCALE)
    assert np.array_equal(k1.cpu().numpy(), rk) and np.array_equal(v1.cpu().numpy(), rv)
    ref = oracle_fp8(inp, fp8.dequantize(rk, K_SCALE), fp8.dequantize(rv, V_SCALE))
    compare(o2, ref, "bf16", what="fp8 decode_append")


def test_fp8_full_bench_workload_sampled():
    """The Qwen-shaped bench workload (64 sequences, 20000-block pool) on E4M3
    caches in the launch bench.py times, checked on sampled (sequence, head)
    pairs."""
    inp = I.generate(I.CONFIGS["qwen7b_gqa_bf16"])
    kq, vq, _, _ = fp8_inputs(inp)
    out = run_fp8(inp, kq, vq)
    rng = np.random.default_rng(5)
    pairs = sorted({(int(b), int(h)) for b, h in zip(rng.integers(0, 64, 48),
                                                      rng.integers(0, 28, 48))})
    used = sorted({b for b, _ in pairs})
    # dequantise only the blocks the sampled sequences read
    blocks = np.unique(np.concatenate([inp.block_tables[b].numpy() for b in used]))
    blocks = blocks[blocks >= 0]
    kdq = np.zeros(kq.shape, dtype=np.float64)
    vdq = np.zeros(vq.shape, dtype=np.float64)
    kdq[blocks] = fp8.dequantize(kq[blocks], K_SCALE)
    vdq[blocks] = fp8.dequantize(vq[blocks], V_SCALE)
    compare(out, oracle_fp8(inp, kdq, vdq, pairs), "bf16", pairs=pairs, what="fp8 bench workload")


@pytest.mark.parametrize("D", [48, 256])
def test_fp8_cache_write_other_head_dims(D):
    """head_dim 48 (a multiple of 16 that is not a power of two) and 256."""
    T, H_kv, BS, N = 100, 3, 32, 16
    g = torch.Generator().manual_seed(D)
    key = (torch.randn(T, H_kv, D, generator=g) * 3).to(torch.bfloat16)
    value = (torch.randn(T, H_kv, D, generator=g) * 9).to(torch.bfloat16)
    slots = np.random.default_rng(D).choice(N * BS, size=T, replace=False).astype(np.int64)
    kc = torch.full((N, H_kv, BS, D), 0x3C, dtype=torch.uint8)
    dk, dv = kc.to(DEV), kc.to(DEV)
    ops.reshape_and_cache_fp8(key.to(DEV), value.to(DEV), dk, dv,
                              torch.from_numpy(slots).to(DEV), K_SCALE, V_SCALE)
    torch.cuda.synchronize()
    rk, rv = fp8.reshape_and_cache_fp8(key.float().numpy(), value.float().numpy(), kc.numpy(),
                                       kc.numpy(), slots, K_SCALE, V_SCALE)
    assert np.array_equal(dk.cpu().numpy(), rk)
    assert np.array_equal(dv.cpu().numpy(), rv)
