"""Long histories on the 8-bit caches and in verify mode: the long-context
workload (4 sequences of 32768 / 65536 / 98304 / 131072 tokens, block size 32,
8 KV heads serving 32 query heads, shuffled tables over a 12288-block pool).
The balanced schedule cuts each of these histories into many pieces across
workgroups; the fixed schedule into 1024-token partitions.  Checked on
sampled (sequence, head) pairs of every sequence against the float64 oracle
([KV-principles] §3.3 asks for quantised caches to be judged on long
sequences).

Over tens of thousands of random tokens plain N(0, 1) queries spread the
attention so evenly that every output is close to 0 (about 1e-3), where a
piece left out or counted twice would still pass a 2e-2 absolute
tolerance.  The queries are therefore scaled (FP8 x 8, bf16 x 4; INT8 codes
are large enough as they are) and rounded to bf16 again: attention then
concentrates on a few dozen tokens scattered over the whole history and the
outputs are of order 0.1 to 0.5.

The 8-bit pools are seeded random codes drawn here on the host (every finite
E4M3 code of magnitude 0.5 .. 120 with a random sign; INT8 codes in
[-127, 127]), so no oracle input comes from the library; the oracle reads
the sampled sequences' blocks dequantised into a compact pool of their own
(a test-side re-layout: the oracle's result does not depend on where a block
lives)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8, int8
from gpu_util import DEV, compare
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

CFG = I.CONFIGS["long_ctx_bf16"]
# every sequence, query heads of several GQA groups
PAIRS = [(0, 3), (1, 17), (2, 30), (3, 0), (3, 13), (3, 31)]
SCALES = {"fp8": (1.0 / 64, 1.0 / 48), "int8": (1.0 / 24, 1.0 / 20)}
Q_GAIN = {"fp8": 8.0, "int8": 1.0, "bf16": 4.0}
CODEC = {"fp8": fp8, "int8": int8}


@pytest.fixture(scope="module")
def work():
    return I.generate(CFG, new_tokens_at="last")


def gained(inp, fmt):
    """The workload with its queries scaled by Q_GAIN[fmt] (rounded to bf16)."""
    q = (inp.query.float() * Q_GAIN[fmt]).to(inp.query.dtype)
    return dataclasses.replace(inp, query=q)


def random_codes(fmt, shape, seed):
    rng = np.random.default_rng(seed)
    if fmt == "fp8":
        mag = rng.integers(0x30, 0x70, size=shape, dtype=np.uint8)   # 0.5 .. 120, no NaN
        return mag | (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7)
    return rng.integers(-127, 128, size=shape, dtype=np.int64).astype(np.int8).view(np.uint8)


def compact(bt, cl, seqs, BS):
    """The blocks the sequences `seqs` read, and their tables remapped into a
    compact pool of just those blocks (other rows -1, lengths 0)."""
    blocks = np.unique(np.concatenate(
        [bt[b, :-(-int(cl[b]) // BS)] for b in seqs])).astype(np.int64)
    where = {int(p): i for i, p in enumerate(blocks)}
    bt2 = np.full_like(bt, -1)
    cl2 = np.zeros_like(cl)
    for b in seqs:
        n = -(-int(cl[b]) // BS)
        bt2[b, :n] = [where[int(p)] for p in bt[b, :n]]
        cl2[b] = cl[b]
    return blocks, bt2.astype(np.int64), cl2.astype(np.int64)


def oracle_8bit(fmt, inp, kq, vq, pairs):
    """The oracle on the dequantised codes, one sampled (sequence, head) at a
    time: its query head against its KV head's codes, from a compact pool of
    that sequence's blocks."""
    ks, vs = SCALES[fmt]
    bt = inp.block_tables.numpy()
    cl = inp.context_lens.numpy()
    G = CFG.num_heads // CFG.num_kv_heads
    out = np.full(tuple(inp.query.shape), np.nan)
    for b, h in pairs:
        blocks, bt2, cl2 = compact(bt, cl, [b], CFG.block_size)
        kdq = CODEC[fmt].dequantize(kq[blocks][:, [h // G]], ks)
        vdq = CODEC[fmt].dequantize(vq[blocks][:, [h // G]], vs)
        q1 = inp.query[b:b + 1, [h]].float().numpy()
        out[b, h] = oracle.decode_contiguous(q1, kdq, vdq, bt2[b:b + 1], cl2[b:b + 1],
                                             CFG.scale)[0, 0]
    return out


def check(out, ref, pairs, what):
    """Parity at the stated tolerance, on references large enough for it to
    mean something (see the module docstring)."""
    idx = tuple(np.array(pairs).T)
    assert np.mean(np.abs(ref[idx])) > 0.03, "%s: outputs too small to discriminate" % what
    compare(out, ref, "bf16", pairs=pairs, what=what)


def decode_8bit(fmt, q, kq, vq, bt, cl, **kw):
    ks, vs = SCALES[fmt]
    f = ops.paged_attention_decode_fp8 if fmt == "fp8" else ops.paged_attention_decode_i8
    return f(q, kq, vq, bt, cl, ks, vs, **kw)


def device_codes(fmt, c):
    t = torch.from_numpy(c).to(DEV)
    return t if fmt == "fp8" else t.view(torch.int8)


@pytest.mark.parametrize("partition_size", [0, 1024])
@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_long_context_8bit_decode(work, fmt, partition_size):
    work = gained(work, fmt)
    shape = tuple(work.key_cache.shape)
    kq = random_codes(fmt, shape, 31)
    vq = random_codes(fmt, shape, 32)
    print("long context %s decode, partition_size %d" % (fmt, partition_size), flush=True)
    out = decode_8bit(fmt, work.query.to(DEV), device_codes(fmt, kq), device_codes(fmt, vq),
                      work.block_tables.to(DEV), work.context_lens.to(DEV),
                      partition_size=partition_size)
    torch.cuda.synchronize()
    ref = oracle_8bit(fmt, work, kq, vq, PAIRS)
    check(out, ref, PAIRS, "%s long context P=%d" % (fmt, partition_size))


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_long_context_8bit_decode_append(work, fmt):
    """The fused append (each sequence's newest token quantised into its
    slot by the decode kernel) equals the cache write followed by the decode,
    bit for bit, caches included; the written codes are the oracle's, and
    the output matches the oracle on the updated caches."""
    work = gained(work, fmt)
    ks, vs = SCALES[fmt]
    shape = tuple(work.key_cache.shape)
    kq = random_codes(fmt, shape, 41)
    vq = random_codes(fmt, shape, 42)
    q = work.query.to(DEV)
    bt, cl = work.block_tables.to(DEV), work.context_lens.to(DEV)
    nk, nv = work.new_key.to(DEV), work.new_value.to(DEV)
    k1, v1 = device_codes(fmt, kq), device_codes(fmt, vq)
    k2, v2 = k1.clone(), v1.clone()
    write = ops.reshape_and_cache_fp8 if fmt == "fp8" else ops.reshape_and_cache_i8
    append = ops.decode_append_fp8 if fmt == "fp8" else ops.decode_append_i8
    write(nk, nv, k1, v1, work.slot_mapping.to(DEV), ks, vs)
    o1 = decode_8bit(fmt, q, k1, v1, bt, cl)
    o2 = append(q, nk, nv, k2, v2, bt, cl, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(o1, o2)
    w = fp8.reshape_and_cache_fp8 if fmt == "fp8" else int8.reshape_and_cache_i8
    rk, rv = w(work.new_key.float().numpy(), work.new_value.float().numpy(), kq, vq,
               work.slot_mapping.numpy(), ks, vs)
    got_k = k1.view(torch.uint8).cpu().numpy()
    got_v = v1.view(torch.uint8).cpu().numpy()
    assert np.array_equal(got_k, rk) and np.array_equal(got_v, rv)
    check(o2, oracle_8bit(fmt, work, rk, rv, PAIRS), PAIRS, "%s long context decode_append" % fmt)


@pytest.mark.parametrize("q_len,partition_size", [(2, 0), (4, 0), (3, 1024)])
def test_long_context_verify(work, q_len, partition_size):
    """Verify rows: q_len newest tokens of each long history, each row
    causal among them, on sampled (row, head) pairs."""
    S, H, D = work.query.shape
    TQ = S * q_len
    g = torch.Generator().manual_seed(q_len)
    qv = (torch.randn(TQ, H, D, generator=g) * Q_GAIN["bf16"]).to(torch.bfloat16)
    qs = torch.arange(0, TQ + 1, q_len, dtype=torch.int32)
    out = ops.paged_attention_verify(qv.to(DEV), work.key_cache.to(DEV),
                                     work.value_cache.to(DEV), work.block_tables.to(DEV),
                                     work.context_lens.to(DEV), qs.to(DEV), q_len,
                                     partition_size=partition_size)
    torch.cuda.synchronize()
    rows = [(b * q_len + i, h) for b, h in PAIRS for i in (0, q_len - 1)]
    # the oracle per sampled (sequence, head): that sequence's blocks and KV
    # head in a compact pool; row i attends the L_b - q_len + i + 1 oldest
    # positions
    bt = work.block_tables.numpy()
    cl = work.context_lens.numpy()
    G = H // CFG.num_kv_heads
    ref = np.full((TQ, H, D), np.nan)
    for b, h in PAIRS:
        blocks, bt2, cl2 = compact(bt, cl, [b], CFG.block_size)
        idx = torch.from_numpy(blocks)
        kc = work.key_cache[idx][:, [h // G]].float().numpy()
        vc = work.value_cache[idx][:, [h // G]].float().numpy()
        one = oracle.decode_verify(qv[b * q_len:(b + 1) * q_len][:, [h]].float().numpy(), kc, vc,
                                   bt2[b:b + 1], cl2[b:b + 1], np.array([0, q_len]), CFG.scale)
        for i in (0, q_len - 1):
            ref[b * q_len + i, h] = one[i, 0]
    check(out, ref, rows, "verify long context q=%d P=%d" % (q_len, partition_size))
