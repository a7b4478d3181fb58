"""Helpers for the GPU parity tests: device upload, oracle inputs, and the
element-wise comparison at the stated tolerances.

Tolerances: float32 inputs, max |o_gpu - o_ref| <= 1e-5; bf16/fp16 inputs
(float32 accumulation), |o_gpu - o_ref| <= 2e-2 + 1e-2 |o_ref| element-wise.
"""

import math

import numpy as np
import torch

from paged_kv_decode_attention_amd import inputs as I

TOL = {"f32": (1e-5, 0.0), "f16": (2e-2, 1e-2), "bf16": (2e-2, 1e-2)}
DEV = "cuda:0"


def upload(inp):
    return dict(
        query=inp.query.to(DEV), key_cache=inp.key_cache.to(DEV),
        value_cache=inp.value_cache.to(DEV), block_tables=inp.block_tables.to(DEV),
        context_lens=inp.context_lens.to(DEV), new_key=inp.new_key.to(DEV),
        new_value=inp.new_value.to(DEV), slot_mapping=inp.slot_mapping.to(DEV))


def oracle_inputs(inp):
    """The exact stored values, widened without rounding (float32 holds every
    bf16/fp16 value); the oracle upcasts to float64 itself."""
    return (inp.query.float().numpy(), inp.key_cache.float().numpy(),
            inp.value_cache.float().numpy(), inp.block_tables.numpy().astype(np.int64),
            inp.context_lens.numpy().astype(np.int64), inp.cfg.scale)


def compare(out_gpu, ref, dtype, pairs=None, what=""):
    """Element-wise check; returns (max_abs, max_rel, worst index)."""
    got = out_gpu.detach().float().cpu().numpy().astype(np.float64)
    if pairs is not None:
        idx = tuple(np.array(pairs).T)
        got, ref = got[idx], ref[idx]
    atol, rtol = TOL[dtype]
    err = np.abs(got - ref)
    bound = atol + rtol * np.abs(ref)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    rel = err / np.maximum(np.abs(ref), 1e-30)
    ok = np.all(err <= bound)
    msg = "%s: max_abs %.3g max_rel %.3g worst %s got %r ref %r" % (
        what, err.max(), rel.max(), worst, got[worst], ref[worst])
    print(msg, flush=True)
    assert ok, msg
    return float(err.max()), float(rel.max()), worst


def small_config(dtype="bf16", H_kv=2, G=7, D=128, BS=16, lens=(1, 15, 16, 17, 100, 513),
                 seed=7, extra_blocks=8, std=1.0):
    nblk = sum(-(-L // BS) for L in lens)
    W = max(1, max(-(-L // BS) for L in lens))
    return I.DecodeConfig(
        name="small", num_seqs=len(lens), num_heads=H_kv * G, num_kv_heads=H_kv,
        head_dim=D, block_size=BS, num_blocks=nblk + extra_blocks, max_blocks_per_seq=W,
        dtype=dtype, value_std=std, lens_kind="list", lens_args=tuple(lens), seed=seed)


def same_history_other_layout(inp, block_size, seed):
    """The same logical K/V histories stored under a fresh shuffled table,
    possibly with another block size (a test-side re-layout)."""
    cfg = inp.cfg
    L = inp.context_lens.numpy()
    BS0 = cfg.block_size
    bt0 = inp.block_tables.numpy()
    nblk = [-(-int(x) // block_size) for x in L]
    N = sum(nblk) + 5
    W = max(1, max(nblk))
    rng = np.random.default_rng(seed)
    perm = rng.permutation(N)
    kc = torch.full((N, cfg.num_kv_heads, block_size, cfg.head_dim), float("nan"),
                    dtype=inp.key_cache.dtype)
    vc = kc.clone()
    bt = np.full((len(L), W), -1, dtype=np.int32)
    cur = 0
    for b, Lb in enumerate(L.tolist()):
        bt[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]
        for pos in range(Lb):
            src = bt0[b, pos // BS0]
            dst = bt[b, pos // block_size]
            kc[dst, :, pos % block_size] = inp.key_cache[src, :, pos % BS0]
            vc[dst, :, pos % block_size] = inp.value_cache[src, :, pos % BS0]
    return kc, vc, torch.from_numpy(bt)
