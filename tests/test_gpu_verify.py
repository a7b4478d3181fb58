"""Verify mode on the GPU (several new query tokens per sequence, causal
among them) against the float64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, compare, small_config
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

RAGGED = (1, 15, 16, 17, 31, 33, 100, 513)


def verify_inputs(cfg, qlens, seed=3):
    inp = I.poison_unread(I.generate(cfg))
    rng = np.random.default_rng(seed)
    qs = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    H, D = cfg.num_heads, cfg.head_dim
    q = torch.from_numpy(rng.standard_normal((int(qs[-1]), H, D)).astype(np.float32)).to(
        inp.query.dtype)
    return inp, q, qs


def oracle_verify(inp, q, qs):
    return oracle.decode_verify(q.float().numpy(), inp.key_cache.float().numpy(),
                                inp.value_cache.float().numpy(),
                                inp.block_tables.numpy().astype(np.int64),
                                inp.context_lens.numpy().astype(np.int64), qs, inp.cfg.scale)


def run_verify(inp, q, qs, max_q, kernel=ops.KERNEL_AUTO, partition_size=0):
    prev = ops.select_kernel(kernel)
    try:
        out = ops.paged_attention_verify(
            q.to(DEV), inp.key_cache.to(DEV), inp.value_cache.to(DEV), inp.block_tables.to(DEV),
            inp.context_lens.to(DEV), torch.from_numpy(qs).to(DEV), max_q,
            partition_size=partition_size)
        torch.cuda.synchronize()
    finally:
        ops.select_kernel(prev)
    return out


CASES = [("bf16", 2, 7, 128, 16, ops.KERNEL_MFMA), ("f16", 2, 4, 128, 32, ops.KERNEL_MFMA),
         ("bf16", 2, 7, 128, 16, ops.KERNEL_GENERIC), ("f32", 2, 1, 64, 16, ops.KERNEL_AUTO)]


@pytest.mark.parametrize("partition_size", [0, 64])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-hkv%d-g%d-d%d-bs%d-k%d" % c)
def test_verify_parity(case, partition_size):
    dtype, H_kv, G, D, BS, kernel = case
    cfg = small_config(dtype, H_kv, G, D, BS, RAGGED)
    # q_b <= L_b, except the first sequence (L = 1, q = 2): its rows are NaN
    qlens = [2, 4, 1, 6, 3, 5, 8, 4]
    inp, q, qs = verify_inputs(cfg, qlens)
    out = run_verify(inp, q, qs, 8, kernel, partition_size)
    ref = oracle_verify(inp, q, qs)
    assert torch.isnan(out[:2].float()).all()
    compare(out[2:], ref[2:], dtype, what="verify %s P=%d" % (case, partition_size))


# Matrix-core verify groups up to 16 // G query rows of a sequence into one
# pass (their (row, head) pairs are the MFMA's 16 columns, each with its own
# causal end), or 32 // G with two column tiles when max_query_len * G > 16
# (head_dim 64 and 128; the cases below pass max_query_len 17).  Lengths put a column's end on a 32-token chunk boundary
# (L_b - q_b + i + 1 = 32 k), so that some chunk (a piece of its own when the
# work list is short, or a partition at P = 32) holds no token of that column
# and leaves an empty state for the merge.
# The sequence of length 3 has q = 5 > L: its rows are NaN.
COL_LENS = (33, 34, 65, 66, 97, 40, 2, 513, 8, 3, 129)
COL_QLENS = (2, 3, 2, 3, 2, 8, 2, 5, 8, 5, 17)
COL_CASES = [("bf16", 2, 7, 128, 16), ("f16", 2, 4, 128, 32), ("bf16", 4, 1, 128, 16),
             ("bf16", 1, 16, 128, 64), ("bf16", 2, 3, 128, 16), ("f16", 1, 8, 128, 16),
             ("bf16", 2, 5, 128, 32), ("bf16", 2, 7, 64, 16), ("f16", 2, 2, 64, 32),
             ("bf16", 2, 7, 256, 16), ("bf16", 1, 4, 256, 64), ("bf16", 2, 7, 128, 8),
             ("bf16", 1, 20, 128, 16), ("f16", 1, 32, 64, 16)]


@pytest.mark.parametrize("partition_size", [0, 64])
@pytest.mark.parametrize("case", COL_CASES, ids=lambda c: "%s-hkv%d-g%d-d%d-bs%d" % c)
def test_verify_columns_parity(case, partition_size):
    dtype, H_kv, G, D, BS = case
    cfg = small_config(dtype, H_kv, G, D, BS, COL_LENS)
    inp, q, qs = verify_inputs(cfg, list(COL_QLENS), seed=11)
    out = run_verify(inp, q, qs, 17, ops.KERNEL_MFMA, partition_size)
    ref = oracle_verify(inp, q, qs)
    bad = np.isnan(ref).any(axis=(1, 2))          # the rows of the L < q sequence
    assert bad.sum() == 5
    assert torch.isnan(out[torch.from_numpy(bad)].float()).all()
    compare(out[torch.from_numpy(~bad)], ref[~bad], dtype,
            what="verify columns %s P=%d" % (case, partition_size))


@pytest.mark.parametrize("partition_size", [0, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 5])
def test_verify_one_column_tile(G, partition_size):
    """max_query_len * G <= 16: one column tile, 16 // G rows per group
    (with max_query_len = 16 // G, every sequence is one group)."""
    u = 16 // G
    lens = (33, 34, 65, 66, 97, 40, 513, 129, 16)
    qlens = [min(u, x) for x in (2, 3, 1, 16, 2, 8, 5, 16, 7)]
    cfg = small_config("bf16", 2, G, 128, 16, lens)
    inp, q, qs = verify_inputs(cfg, qlens, seed=13)
    out = run_verify(inp, q, qs, u, ops.KERNEL_MFMA, partition_size)
    compare(out, oracle_verify(inp, q, qs), "bf16",
            what="verify one tile G=%d P=%d" % (G, partition_size))


@pytest.mark.parametrize("G,BS", [(7, 16), (1, 16)])
def test_verify_columns_fixed_partition_boundary(G, BS):
    """P = 32: every 32-token partition is its own state; columns whose causal
    end is a multiple of 32 have an empty trailing partition."""
    cfg = small_config("bf16", 2, G, 128, BS, COL_LENS)
    inp, q, qs = verify_inputs(cfg, list(COL_QLENS), seed=12)
    out = run_verify(inp, q, qs, 17, ops.KERNEL_MFMA, 32)
    ref = oracle_verify(inp, q, qs)
    bad = np.isnan(ref).any(axis=(1, 2))
    assert bad.sum() == 5
    assert torch.isnan(out[torch.from_numpy(bad)].float()).all()
    compare(out[torch.from_numpy(~bad)], ref[~bad], "bf16", what="verify columns P=32 G=%d" % G)


def test_verify_single_query_equals_decode():
    cfg = small_config("bf16", 2, 7, 128, 16, RAGGED)
    inp, _, _ = verify_inputs(cfg, [1] * len(RAGGED))
    qs = np.arange(len(RAGGED) + 1, dtype=np.int32)
    d = dict(q=inp.query.to(DEV), kc=inp.key_cache.to(DEV), vc=inp.value_cache.to(DEV),
             bt=inp.block_tables.to(DEV), cl=inp.context_lens.to(DEV))
    a = ops.paged_attention_decode(d["q"], d["kc"], d["vc"], d["bt"], d["cl"])
    b = ops.paged_attention_verify(d["q"], d["kc"], d["vc"], d["bt"], d["cl"],
                                   torch.from_numpy(qs).to(DEV), 1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_verify_rows_beyond_max_query_len_are_nan():
    cfg = small_config("bf16", 2, 7, 128, 16, (100, 200))
    inp, q, qs = verify_inputs(cfg, [3, 5])
    out = run_verify(inp, q, qs, 4)           # the second sequence has q = 5 > 4
    ref = oracle_verify(inp, q, qs)
    assert torch.isnan(out[3:].float()).all()
    compare(out[:3], ref[:3], "bf16", what="verify within bound")


def test_verify_bench_workload_q4_sampled():
    cfg = I.CONFIGS["qwen7b_gqa_bf16"]
    inp, q, qs = verify_inputs(cfg, [4] * cfg.num_seqs)
    out = run_verify(inp, q, qs, 4)
    rows = list(range(0, 256, 17))
    ref = np.full((q.shape[0], cfg.num_heads, cfg.head_dim), np.nan)
    sub_q = q.float().numpy()
    kc, vc = inp.key_cache.float().numpy(), inp.value_cache.float().numpy()
    for r in rows:
        b = r // 4
        sel = oracle.decode_verify(sub_q[4 * b:4 * b + 4], kc, vc,
                                   inp.block_tables.numpy()[b:b + 1].astype(np.int64),
                                   inp.context_lens.numpy()[b:b + 1].astype(np.int64),
                                   np.array([0, 4]), cfg.scale)
        ref[r] = sel[r - 4 * b]
    compare(out[rows], ref[rows], "bf16", what="verify bench workload q=4")


@pytest.mark.parametrize("G,D", [(7, 128), (4, 256)])
def test_verify_balanced_row_limit(G, D):
    """2048 query rows on the balanced schedule, the most it takes: the
    decode kernel's prologue then holds the prefix table, the rows' lengths
    and their row map in LDS beside the edge pieces (two column tiles at
    head_dim 128, the largest edge LDS)."""
    nseq = 512
    lens = tuple(33 + (7 * i) % 90 for i in range(nseq))
    cfg = small_config("bf16", 2, G, D, 16, lens)
    inp, q, qs = verify_inputs(cfg, [4] * nseq, seed=21)
    out = run_verify(inp, q, qs, 4, ops.KERNEL_MFMA)
    compare(out, oracle_verify(inp, q, qs), "bf16", what="verify 2048 rows G=%d D=%d" % (G, D))


@pytest.mark.parametrize("nsrc", [4096, 4097])
def test_verify_many_sequences_few_queries(nsrc):
    """Sequences without query rows.  The balanced decode kernel stages every
    sequence's query start and length in LDS to compute the row map (up to
    4096 sequences); with more, the row map is written to memory first and
    the fixed schedule reads it."""
    lens = tuple(5 + (i * 13) % 60 for i in range(nsrc))
    rng = np.random.default_rng(nsrc)
    qlens = [0] * nsrc
    for b in rng.choice(nsrc, 40, replace=False):
        qlens[int(b)] = int(min(lens[int(b)], rng.integers(1, 5)))
    qlens[nsrc - 1] = 2                       # the last sequence has rows too
    cfg = small_config("bf16", 1, 4, 64, 16, lens)
    inp, q, qs = verify_inputs(cfg, qlens, seed=22)
    out = run_verify(inp, q, qs, 4, ops.KERNEL_MFMA)
    compare(out, oracle_verify(inp, q, qs), "bf16", what="verify %d sequences" % nsrc)
