"""Decode parity on the GPU: the HIP kernels, called through the C ABI,
against the float64 oracle, element by element, on the same seeded inputs.

Every pool slot no history token occupies is NaN (tail slots of last blocks,
blocks no table references) and unused table entries are -1, so any read
past the history shows up as a non-finite output.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, compare, oracle_inputs, same_history_other_layout, small_config, upload
from paged_kv_decode_attention_amd import inputs as I
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

RAGGED = (1, 15, 16, 17, 31, 33, 100, 513)


def run_decode(d, kernel=ops.KERNEL_AUTO, partition_size=0, **kw):
    prev = ops.select_kernel(kernel)
    try:
        out = ops.paged_attention_decode(d["query"], d["key_cache"], d["value_cache"],
                                         d["block_tables"], d["context_lens"],
                                         partition_size=partition_size, **kw)
        torch.cuda.synchronize()
    finally:
        ops.select_kernel(prev)
    return out


def oracle_ref(inp, pairs=None):
    return oracle.decode_contiguous(*oracle_inputs(inp), pairs=pairs)


# ---------------------------------------------------------------- small shapes

SMALL_CASES = [
    # dtype, H_kv, G, D, BS, kernel
    ("bf16", 2, 7, 128, 16, ops.KERNEL_MFMA),
    ("bf16", 2, 7, 128, 16, ops.KERNEL_GENERIC),
    ("f16", 2, 4, 128, 16, ops.KERNEL_MFMA),
    ("f16", 2, 4, 128, 32, ops.KERNEL_MFMA),
    ("bf16", 3, 1, 128, 32, ops.KERNEL_MFMA),
    ("bf16", 1, 16, 128, 16, ops.KERNEL_MFMA),
    ("bf16", 2, 8, 128, 32, ops.KERNEL_MFMA),
    ("bf16", 2, 20, 128, 16, ops.KERNEL_AUTO),      # G 17..32: two column tiles
    ("bf16", 1, 32, 128, 32, ops.KERNEL_MFMA),
    ("f16", 2, 17, 64, 16, ops.KERNEL_MFMA),
    ("bf16", 1, 24, 128, 8, ops.KERNEL_MFMA),
    ("bf16", 1, 40, 128, 16, ops.KERNEL_AUTO),      # G > 32: two passes of 20 heads
    ("bf16", 1, 20, 256, 16, ops.KERNEL_AUTO),      # G > 16 at head_dim 256: two passes of 10
    ("bf16", 1, 64, 128, 16, ops.KERNEL_MFMA),      # two passes of 32 (two column tiles)
    ("f16", 2, 48, 64, 32, ops.KERNEL_MFMA),        # two passes of 24
    ("bf16", 1, 32, 256, 8, ops.KERNEL_MFMA),       # two passes of 16 at head_dim 256
    ("bf16", 2, 96, 128, 16, ops.KERNEL_MFMA),      # three passes of 32
    ("bf16", 1, 37, 128, 16, ops.KERNEL_AUTO),      # passes of 19 and 18 heads
    ("f16", 2, 33, 64, 16, ops.KERNEL_MFMA),        # passes of 17 and 16
    ("bf16", 1, 37, 256, 16, ops.KERNEL_MFMA),      # passes of 13, 13 and 11 at head_dim 256
    ("bf16", 1, 17, 256, 8, ops.KERNEL_AUTO),       # passes of 9 and 8, block size 8
    ("bf16", 2, 70, 128, 32, ops.KERNEL_MFMA),      # passes of 24, 24 and 22
    ("f16", 1, 101, 64, 64, ops.KERNEL_AUTO),       # passes of 26, 26, 26 and 23
    ("bf16", 1, 64, 128, 16, ops.KERNEL_GENERIC),
    ("f16", 2, 3, 64, 16, ops.KERNEL_AUTO),         # head_dim 64: matrix-core kernel
    ("bf16", 2, 5, 64, 32, ops.KERNEL_GENERIC),
    ("bf16", 2, 7, 64, 16, ops.KERNEL_MFMA),
    ("bf16", 3, 1, 64, 32, ops.KERNEL_MFMA),
    ("f16", 1, 16, 64, 64, ops.KERNEL_MFMA),
    ("bf16", 2, 8, 64, 16, ops.KERNEL_MFMA),
    ("f32", 2, 1, 64, 16, ops.KERNEL_AUTO),         # float32 rows: f32 matrix cores
    ("f32", 2, 7, 128, 16, ops.KERNEL_MFMA),
    ("f32", 1, 16, 64, 8, ops.KERNEL_MFMA),         # block size 8: per-lane addresses
    ("f32", 2, 4, 128, 64, ops.KERNEL_AUTO),
    ("f32", 1, 20, 128, 32, ops.KERNEL_AUTO),       # passes of 10 heads
    ("f32", 3, 5, 64, 32, ops.KERNEL_MFMA),
    ("f32", 2, 4, 128, 32, ops.KERNEL_GENERIC),
    ("f32", 1, 12, 128, 16, ops.KERNEL_GENERIC),
    ("f32", 2, 7, 64, 16, ops.KERNEL_GENERIC),      # 8-head workgroups: block fold
    ("f32", 1, 8, 256, 32, ops.KERNEL_AUTO),        # head_dim 256: vector ALU, block fold
    ("f32", 1, 13, 64, 8, ops.KERNEL_GENERIC),      # block fold + a 5-head workgroup
    # block sizes 8 and 64, head_dim 256
    ("bf16", 2, 7, 128, 64, ops.KERNEL_MFMA),
    ("f16", 2, 4, 128, 8, ops.KERNEL_AUTO),         # block size 8: matrix-core kernel
    ("bf16", 2, 7, 128, 8, ops.KERNEL_MFMA),
    ("bf16", 1, 8, 64, 8, ops.KERNEL_MFMA),
    ("f16", 2, 4, 256, 8, ops.KERNEL_MFMA),
    ("bf16", 2, 7, 128, 8, ops.KERNEL_GENERIC),
    ("bf16", 2, 4, 256, 16, ops.KERNEL_AUTO),       # head_dim 256: matrix-core kernel
    ("f16", 2, 7, 256, 32, ops.KERNEL_MFMA),
    ("bf16", 1, 16, 256, 64, ops.KERNEL_MFMA),
    ("bf16", 3, 1, 256, 16, ops.KERNEL_MFMA),
    ("bf16", 2, 4, 256, 16, ops.KERNEL_GENERIC),
    ("f32", 2, 2, 256, 64, ops.KERNEL_GENERIC),
    ("bf16", 1, 8, 64, 8, ops.KERNEL_GENERIC),
    ("f16", 2, 3, 64, 64, ops.KERNEL_GENERIC),
]


@pytest.mark.parametrize("partition_size", [0, 32, 64, 256])
@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: "%s-hkv%d-g%d-d%d-bs%d-k%d" % c)
def test_small_parity(case, partition_size):
    dtype, H_kv, G, D, BS, kernel = case
    if partition_size and partition_size % BS:
        pytest.skip("partition not a multiple of the block size")
    inp = I.poison_unread(I.generate(small_config(dtype, H_kv, G, D, BS, RAGGED)))
    out = run_decode(upload(inp), kernel, partition_size)
    compare(out, oracle_ref(inp), dtype, what="small %s P=%d" % (case, partition_size))


def test_kernels_agree():
    inp = I.poison_unread(I.generate(small_config("bf16", 4, 7, 128, 16, RAGGED, seed=3)))
    d = upload(inp)
    a = run_decode(d, ops.KERNEL_MFMA).float()
    b = run_decode(d, ops.KERNEL_GENERIC).float()
    assert torch.all(torch.abs(a - b) <= 2e-2 + 1e-2 * torch.abs(b))


def test_single_token_history_is_v0_exactly():
    for dtype, D, kernel in (("bf16", 128, ops.KERNEL_MFMA), ("f16", 128, ops.KERNEL_MFMA),
                             ("bf16", 64, ops.KERNEL_MFMA), ("bf16", 256, ops.KERNEL_MFMA),
                             ("f32", 64, ops.KERNEL_GENERIC), ("f32", 128, ops.KERNEL_MFMA),
                             ("f32", 64, ops.KERNEL_MFMA),
                             ("bf16", 128, ops.KERNEL_GENERIC)):
        inp = I.generate(small_config(dtype, 2, 4, D, 16, (1, 1, 1)))
        out = run_decode(upload(inp), kernel).cpu()
        for b in range(3):
            pb = int(inp.block_tables[b, 0])
            for h in range(8):
                v0 = inp.value_cache[pb, h // 4, 0]
                assert torch.equal(out[b, h], v0), (dtype, kernel, b, h)


def test_empty_history_gives_zeros():
    for kernel in (ops.KERNEL_MFMA, ops.KERNEL_GENERIC):
        inp = I.generate(small_config("bf16", 2, 7, 128, 16, (5, 40, 3)))
        inp.context_lens[1] = 0
        out = run_decode(upload(inp), kernel).cpu()
        assert torch.all(out[1] == 0)
        ref = oracle_ref(inp)
        compare(out, ref, "bf16", what="with empty row")


@pytest.mark.parametrize("BS", [16, 8])
def test_invalid_device_data_gives_nan_rows(BS):
    for kernel in (ops.KERNEL_MFMA, ops.KERNEL_GENERIC):
        inp = I.generate(small_config("bf16", 2, 7, 128, BS, (40, 40, 40, 40)))
        inp.context_lens[1] = 10_000          # > max_context_len
        inp.context_lens[2] = -3
        inp.block_tables[3, 1] = 10_000_000   # outside the pool
        out = run_decode(upload(inp), kernel).cpu().float()
        assert torch.isnan(out[1]).all() and torch.isnan(out[2]).all()
        assert torch.isnan(out[3]).all()
        assert torch.isfinite(out[0]).all()


def test_balanced_prologue_many_rows_empty_and_invalid():
    """The balanced schedule with 700 decode rows (the prologue's prefix table
    takes three rows a thread): rows with no history give zeros and rows with
    an invalid length NaN, also past the first 256 rows (each workgroup tests
    rows w, w + 256, ... together); the other rows against the oracle."""
    S = 700
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 48, S)
    lens[1] = 600                         # not a small call: the balanced schedule
    zero_rows = [0, 255, 256, 300, 511, 699]
    bad_rows = [5, 257, 512, 698]
    lens[zero_rows] = 0
    cfg = small_config("bf16", 1, 4, 128, 16, tuple(int(x) for x in lens), extra_blocks=4)
    inp = I.poison_unread(I.generate(cfg))
    good = [r for r in range(S) if r not in zero_rows and r not in bad_rows]
    rows = [1] + [int(r) for r in rng.choice(good[2:], 40, replace=False)]
    pairs = [(b, h) for b in rows for h in range(4)]
    ref = oracle_ref(inp, pairs)
    for i, r in enumerate(bad_rows):
        inp.context_lens[r] = 10_000 if i % 2 == 0 else -3
    out = run_decode(upload(inp), ops.KERNEL_MFMA)
    host = out.cpu().float()
    for r in zero_rows:
        assert torch.all(host[r] == 0), "row %d" % r
    for r in bad_rows:
        assert torch.isnan(host[r]).all(), "row %d" % r
    compare(out, ref, "bf16", pairs=pairs, what="700 rows, empty and invalid ones among them")


def test_permutation_and_block_size_invariance_bitwise():
    inp = I.generate(small_config("bf16", 2, 7, 128, 16, RAGGED, seed=11))
    base = run_decode(upload(inp), ops.KERNEL_MFMA, 256).cpu()
    for bs, seed in ((16, 1), (16, 2), (32, 3)):
        kc, vc, bt = same_history_other_layout(inp, bs, seed)
        d = dict(query=inp.query.to(DEV), key_cache=kc.to(DEV), value_cache=vc.to(DEV),
                 block_tables=bt.to(DEV), context_lens=inp.context_lens.to(DEV))
        out = run_decode(d, ops.KERNEL_MFMA, 256).cpu()
        assert torch.equal(out, base), "layout (bs=%d, seed=%d) changed the result" % (bs, seed)


@pytest.mark.parametrize("D", [128, 64, 256])
def test_balanced_schedule_layout_invariance_bitwise(D):
    """The balanced schedule's work split depends on lengths only, so moving
    the history to other physical blocks, or to blocks of 8, 32 or 64, changes
    no bit."""
    inp = I.generate(small_config("bf16", 2, 7, D, 16, RAGGED + (2000, 3000), seed=12))
    base = run_decode(upload(inp), ops.KERNEL_MFMA, 0).cpu()
    for bs, seed in ((16, 4), (32, 5), (8, 6), (64, 7)):
        kc, vc, bt = same_history_other_layout(inp, bs, seed)
        d = dict(query=inp.query.to(DEV), key_cache=kc.to(DEV), value_cache=vc.to(DEV),
                 block_tables=bt.to(DEV), context_lens=inp.context_lens.to(DEV))
        out = run_decode(d, ops.KERNEL_MFMA, 0).cpu()
        assert torch.equal(out, base), "layout (bs=%d, seed=%d) changed the result" % (bs, seed)


def test_balanced_workspace_reuse_and_all_empty():
    """One workspace, first filled with a junk byte pattern, serves a batch
    with no history at all (every row 0), a full batch and the empty batch
    again: nothing a call leaves behind leaks into the next."""
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_seqs=16, num_blocks=4200)
    inp = I.poison_unread(I.generate(cfg))
    d = upload(inp)
    S, H, D = inp.query.shape
    n = ops.decode_workspace_size(S, H, cfg.num_kv_heads, D, cfg.block_size,
                                  cfg.max_blocks_per_seq * cfg.block_size, 0, inp.query.dtype)
    ws = torch.full((n,), 1, dtype=torch.uint8, device=DEV)
    empty = torch.zeros_like(d["context_lens"])
    for lens, want in ((empty, "zeros"), (d["context_lens"], "oracle"), (empty, "zeros")):
        out = torch.full_like(d["query"], float("nan"))
        ops.paged_attention_decode(d["query"], d["key_cache"], d["value_cache"],
                                   d["block_tables"], lens, out=out, workspace=ws)
        torch.cuda.synchronize()
        if want == "zeros":
            assert torch.all(out == 0)
        else:
            compare(out, oracle_ref(inp), "bf16", what="after an empty batch")


@pytest.mark.parametrize("dtype,G,D,BS,lens", [
    ("bf16", 7, 128, 16, (1, 15, 16, 17, 100, 500)),     # one fixed partition of 512
    ("f16", 4, 64, 8, (3, 64, 65, 200)),
    ("bf16", 20, 128, 32, (31, 32, 33, 250)),             # two column tiles
    ("bf16", 37, 256, 16, (5, 130, 256)),                 # three passes
    ("f32", 7, 128, 16, (1, 40, 300)),                    # float32: vector ALU
])
def test_small_call_single_partition(dtype, G, D, BS, lens):
    """Calls whose histories fit 512 tokens take one fixed partition covering
    every history (one launch, no merge); against the oracle."""
    inp = I.poison_unread(I.generate(small_config(dtype, 2, G, D, BS, lens)))
    P = ops.decode_partition_size(len(lens), 2, G, D, BS, inp.block_tables.shape[1] * BS,
                                  inp.query.dtype)
    assert P >= inp.block_tables.shape[1] * BS
    out = run_decode(upload(inp), ops.KERNEL_AUTO, 0)
    compare(out, oracle_ref(inp), dtype, what="small call %s G=%d D=%d" % (dtype, G, D))


def test_partition_size_invariance():
    inp = I.poison_unread(I.generate(small_config("bf16", 2, 7, 128, 32, (700, 1000, 64))))
    d = upload(inp)
    ref = oracle_ref(inp)
    outs = [run_decode(d, ops.KERNEL_MFMA, P) for P in (32, 64, 128, 512, 1024, 2048)]
    for o in outs:
        compare(o, ref, "bf16", what="partition sweep")


def test_shared_blocks_across_sequences():
    # two sequences read the same physical blocks (a shared prefix)
    inp = I.generate(small_config("bf16", 2, 7, 128, 16, (100, 100, 50)))
    inp.block_tables[1, :4] = inp.block_tables[0, :4]
    out = run_decode(upload(inp), ops.KERNEL_MFMA)
    compare(out, oracle_ref(inp), "bf16", what="shared prefix")


def test_gather_index_math_bit_exact():
    for cfg in (small_config("bf16", 2, 7, 128, 16, RAGGED),
                small_config("f32", 3, 1, 64, 32, (5, 64, 65))):
        inp = I.generate(cfg)
        d = upload(inp)
        kc16 = inp.key_cache.view(torch.int16 if cfg.dtype != "f32" else torch.int32).numpy()
        vc16 = inp.value_cache.view(torch.int16 if cfg.dtype != "f32" else torch.int32).numpy()
        for b, L in enumerate(inp.context_lens.tolist()):
            k, v = ops.debug_gather_kv(d["key_cache"], d["value_cache"], d["block_tables"],
                                       d["context_lens"], b)
            torch.cuda.synchronize()
            view = torch.int16 if cfg.dtype != "f32" else torch.int32
            gk = k.cpu().view(view).numpy()[:, :L]
            gv = v.cpu().view(view).numpy()[:, :L]
            rk, rv = oracle.gather_sequence_kv(kc16, vc16, inp.block_tables[b].numpy(), L)
            assert np.array_equal(gk, rk) and np.array_equal(gv, rv), (cfg.dtype, b)


# ------------------------------------------------ full workloads, bench launch

_FULL = {}


def full_inputs(name):
    if name not in _FULL:
        _FULL.clear()
        inp = I.generate(I.CONFIGS[name])
        _FULL[name] = (inp, upload(inp))
    return _FULL[name]


@pytest.mark.parametrize("name", I.CONFIG_ORDER)
def test_full_config_parity(name):
    inp, d = full_inputs(name)
    out = run_decode(d)
    ref = oracle_ref(inp)
    compare(out, ref, inp.cfg.dtype, what="config %s" % name)


def test_long_context_ragged_tails():
    cfg = I.CONFIGS["long_ctx_bf16"]
    lens = [L - r for L, r in zip(cfg.lens_args, (1, 7, 13, 31))]
    inp = I.poison_unread(I.generate(cfg, lens=lens))
    d = upload(inp)
    pairs = [(b, h) for b in range(4) for h in (0, 5, 13, 31)]
    ref = oracle_ref(inp, pairs)
    for P in (0, 512, 2048):
        out = run_decode(d, partition_size=P)
        compare(out, ref, "bf16", pairs=pairs, what="long ragged P=%d" % P)


@pytest.mark.parametrize("G,L", [(7, 65536 - 5), (4, 131072), (16, 40000)])
def test_one_long_sequence(G, L):
    """One sequence with a long history: on the balanced schedule each of its
    KV heads' histories is cut into tens of pieces (64 at 131072 tokens over
    4 KV heads), which the merge folds in several thread subsets at once;
    checked against the oracle on sampled heads."""
    H_kv = 4 if G != 16 else 2
    cfg = I.with_overrides(I.CONFIGS["long_ctx_bf16"], num_seqs=1, num_heads=H_kv * G,
                           num_kv_heads=H_kv, block_size=16,
                           num_blocks=L // 16 + 64, max_blocks_per_seq=L // 16 + 16)
    inp = I.poison_unread(I.generate(cfg, lens=[L]))
    d = upload(inp)
    pairs = [(0, h) for h in range(0, H_kv * G, max(1, G // 3))]
    ref = oracle_ref(inp, pairs)
    out = run_decode(d)
    compare(out, ref, "bf16", pairs=pairs, what="one sequence of %d tokens, G=%d" % (L, G))


@pytest.mark.parametrize("G,D", [(37, 128), (37, 256), (100, 64)])
def test_uneven_passes_on_the_bench_batch(G, D):
    """A group that splits into unequal passes (19 + 18 heads at head_dim 128,
    13 + 13 + 11 at 256, 4 x 25 at 64 -- even, for contrast) on the bench
    batch's 64 histories of 512 to 4096 tokens: every history is cut across
    workgroups and merged.  Sampled against the oracle at the heads on each
    side of every pass boundary."""
    cfg = I.with_overrides(I.CONFIGS["qwen7b_gqa_bf16"], num_heads=2 * G, num_kv_heads=2,
                           head_dim=D)
    inp = I.poison_unread(I.generate(cfg))
    d = upload(inp)
    cap = 16 if D == 256 else 32
    passes = -(-G // cap)
    pg = -(-G // passes)
    heads = sorted({h for j in range(passes) for h in (j * pg, min(G, (j + 1) * pg) - 1)})
    rng = np.random.default_rng(G + D)
    pairs = [(int(b), kvh * G + h) for b in rng.choice(64, 12, replace=False)
             for kvh in range(2) for h in heads]
    out = run_decode(d)
    compare(out, oracle_ref(inp, pairs), "bf16", pairs=pairs, what="G=%d D=%d" % (G, D))


@pytest.mark.parametrize("D,H_kv", [(128, 4), (64, 8)])
def test_staged_rows_overflow(D, H_kv):
    """Whole histories' output rows go to a per-wavefront LDS stage (75 rows
    at head_dim 128, 200 at 64) and out after the wavefront's last piece;
    with 16 heads a history and 2048 short histories per KV head a
    wavefront finishes more histories than its stage holds, so the rows
    past it are stored directly.  Every sequence checked on two heads, and
    empty histories give zero rows."""
    rng = np.random.default_rng(D + H_kv)
    lens = rng.integers(1, 40, 2048)
    lens[::61] = 0
    lens[3] = 600            # keeps the call off the one-partition path
    cfg = small_config("bf16", H_kv, 16, D, 16, tuple(int(x) for x in lens), extra_blocks=4)
    inp = I.poison_unread(I.generate(cfg))
    out = run_decode(upload(inp), ops.KERNEL_MFMA)
    H = H_kv * 16
    pairs = [(b, int(h)) for b in range(2048) if lens[b] > 0
             for h in rng.choice(H, 2, replace=False)]
    compare(out, oracle_ref(inp, pairs), "bf16", pairs=pairs,
            what="staged rows D=%d H_kv=%d" % (D, H_kv))
    assert torch.all(out[torch.from_numpy(lens == 0)] == 0)


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("S", [2048, 2049])
def test_many_sequences_balanced_limit(S, D):
    """The balanced schedule's prefix table (dynamic LDS, S + 1 ints) at its
    largest, next to 134 KB of edge LDS at head_dim 256; one sequence more
    takes the fixed schedule.  Short ragged histories, some empty, and one of
    600 tokens (a call whose histories all fit 512 tokens would take one
    fixed partition)."""
    rng = np.random.default_rng(S + D)
    lens = rng.integers(0, 48, S)
    lens[::97] = 0
    lens[1] = 600
    cfg = small_config("bf16", 1, 4, D, 16, tuple(int(x) for x in lens), extra_blocks=4)
    inp = I.poison_unread(I.generate(cfg))
    out = run_decode(upload(inp), ops.KERNEL_MFMA)
    rows = np.concatenate([[1], rng.choice(np.arange(2, S), 63, replace=False)])
    pairs = [(int(b), h) for b in rows for h in range(4)]
    compare(out, oracle_ref(inp, pairs), "bf16", pairs=pairs, what="S=%d D=%d" % (S, D))
    assert torch.all(out[torch.from_numpy(lens == 0)] == 0)
