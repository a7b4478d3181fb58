"""Copy-on-write on the GPU: pa_copy_blocks bit-exact against the oracle,
and the whole write side of shared blocks -- the library's pool hands out
slots and copy pairs, pa_copy_blocks and pa_reshape_and_cache store the
tokens, and every sequence then decodes exactly its own logical history."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import DEV, compare
from paged_kv_decode_attention_amd import ops

pytestmark = pytest.mark.gpu

BITS = {torch.float32: torch.int32, torch.float16: torch.int16, torch.bfloat16: torch.int16}


def bits(t):
    return t.detach().cpu().view(BITS[t.dtype]).numpy()


@pytest.mark.parametrize("dtype,H_kv,D,BS", [(torch.float32, 2, 64, 16), (torch.bfloat16, 4, 128, 16),
                                              (torch.float16, 8, 128, 32), (torch.bfloat16, 1, 64, 1)])
def test_copy_blocks_bit_exact(dtype, H_kv, D, BS):
    N = 40
    g = torch.Generator().manual_seed(3)
    kc = torch.randn(N, H_kv, BS, D, generator=g).to(dtype)
    vc = torch.randn(N, H_kv, BS, D, generator=g).to(dtype)
    pairs = [(1, 7), (1, 8), (30, 2), (39, 0), (5, 5), (3, N + 2), (-1, 4)]
    dk, dv = kc.to(DEV), vc.to(DEV)
    ops.copy_blocks(dk, dv, torch.tensor(pairs, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    valid = [(s, d) for s, d in pairs if 0 <= s < N and 0 <= d < N and s != d]
    rk, rv = oracle.copy_blocks(bits(kc), bits(vc), valid)
    assert np.array_equal(bits(dk), rk) and np.array_equal(bits(dv), rv)


def test_copy_on_write_end_to_end():
    rng = np.random.default_rng(21)
    N, BS, H_kv, G, D = 96, 16, 2, 4, 128
    H = H_kv * G
    dtype = torch.bfloat16
    pool = ops.BlockPool(N, BS)
    ref = oracle.BlockPool(N, BS)
    kc = torch.full((N, H_kv, BS, D), float("nan"), dtype=dtype)
    vc = kc.clone()
    dk, dv = kc.to(DEV), vc.to(DEV)
    rk, rv = bits(kc), bits(vc)                 # oracle caches, raw bits
    rows_k, rows_v = [], []                     # K/V row of every token ever appended
    seqs, rids = [], []                         # library ids, oracle ids

    def append(which):
        nonlocal rk, rv
        ids = [seqs[i] for i in which]
        slots, pairs = pool.append(ids)
        new_k = torch.randn(len(ids), H_kv, D).to(dtype)
        new_v = torch.randn(len(ids), H_kv, D).to(dtype)
        if len(pairs):
            ops.copy_blocks(dk, dv, torch.from_numpy(pairs).to(DEV))
        ops.reshape_and_cache(new_k.to(DEV), new_v.to(DEV), dk, dv,
                              torch.from_numpy(slots).to(DEV))
        toks = list(range(len(rows_k), len(rows_k) + len(which)))
        want_slots, want_pairs = ref.append([rids[i] for i in which], toks)
        rows_k.extend(new_k)
        rows_v.extend(new_v)
        assert slots.tolist() == want_slots
        assert pairs.tolist() == [list(p) for p in want_pairs]
        rk, rv = oracle.copy_blocks(rk, rv, want_pairs)
        rk, rv = oracle.reshape_and_cache(bits(new_k), bits(new_v), rk, rv, slots)

    def fork(i):
        seqs.append(pool.fork(seqs[i]))
        rids.append(ref.fork(rids[i]))

    for _ in range(3):
        seqs.append(pool.add_sequence())
        rids.append(ref.add_sequence())
    for step in range(40):                      # prompts of 40 tokens
        append([0, 1, 2])
    fork(0)                                     # 40 % 16 = 8: shared partial tail
    fork(0)
    fork(1)
    for step in range(int(rng.integers(5, 30))):
        live = list(range(len(seqs)))
        rng.shuffle(live)
        append(live[: int(rng.integers(1, len(live) + 1))])
        if step == 7:
            fork(3)                             # fork a branch mid-block
    torch.cuda.synchronize()
    # the device caches hold exactly what the oracle's writes and copies give
    # (slots no sequence holds keep their NaN bits on both sides)
    assert np.array_equal(bits(dk), rk) and np.array_equal(bits(dv), rv)

    S = len(seqs)
    lens = [pool.length(s) for s in seqs]
    W = max(len(ref.table(r)) for r in rids)
    bt = np.full((S, W), -1, dtype=np.int32)
    for b, s in enumerate(seqs):
        t = pool.table(s)
        assert list(t) == ref.table(rids[b])
        bt[b, :len(t)] = t
    q = torch.randn(S, H, D).to(dtype)
    out = ops.paged_attention_decode(q.to(DEV), dk, dv, torch.from_numpy(bt).to(DEV),
                                     torch.tensor(lens, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    # reference: attention over each sequence's logical history, the token
    # rows in the order the oracle pool reads them back
    ref_out = np.zeros((S, H, D))
    scale = 1.0 / np.sqrt(D)
    for b in range(S):
        toks = ref.read(rids[b])
        assert len(toks) == lens[b]
        K = torch.stack([rows_k[t] for t in toks]).double().numpy()    # [L, H_kv, D]
        V = torch.stack([rows_v[t] for t in toks]).double().numpy()
        for h in range(H):
            kvh = h // G
            s = scale * (K[:, kvh] @ q[b, h].double().numpy())
            p = np.exp(s - s.max())
            ref_out[b, h] = (p / p.sum()) @ V[:, kvh]
    compare(out, ref_out, "bf16", what="copy-on-write branches")
