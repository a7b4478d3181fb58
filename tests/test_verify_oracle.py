"""Pins of the verify (several new query tokens per sequence) oracle: a
library special case (torch SDPA with an explicit causal mask, float64), the
q = 1 reduction to decode, brute force, and causality."""

import math

import numpy as np
import torch

import oracle


def make(seed=0, S=3, H=4, H_kv=2, D=16, BS=4, lens=(9, 5, 12), qlens=(3, 1, 4)):
    rng = np.random.default_rng(seed)
    N = sum(-(-L // BS) for L in lens) + 3
    kc = rng.standard_normal((N, H_kv, BS, D))
    vc = rng.standard_normal((N, H_kv, BS, D))
    perm = rng.permutation(N)
    W = max(-(-L // BS) for L in lens)
    bt = np.full((S, W), -1, dtype=np.int64)
    k = 0
    for b, L in enumerate(lens):
        n = -(-L // BS)
        bt[b, :n] = perm[k:k + n]
        k += n
    qs = np.concatenate([[0], np.cumsum(qlens)])
    q = rng.standard_normal((int(qs[-1]), H, D))
    return q, kc, vc, bt, np.array(lens), qs, 1 / math.sqrt(D)


def test_sdpa_with_causal_mask():
    q, kc, vc, bt, cl, qs, scale = make()
    out = oracle.decode_verify(q, kc, vc, bt, cl, qs, scale)
    H, H_kv = q.shape[1], kc.shape[1]
    G = H // H_kv
    for b in range(len(cl)):
        L, q_b = int(cl[b]), int(qs[b + 1] - qs[b])
        K, V = oracle.gather_sequence_kv(kc, vc, bt[b], L)          # [H_kv, L, D]
        Kt = torch.from_numpy(np.repeat(K, G, axis=0))
        Vt = torch.from_numpy(np.repeat(V, G, axis=0))
        Q = torch.from_numpy(q[qs[b]:qs[b + 1]].transpose(1, 0, 2).copy())   # [H, q_b, D]
        t = torch.arange(L)[None, :]
        i = torch.arange(q_b)[:, None]
        mask = t <= (L - q_b + i)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, Kt, Vt, attn_mask=mask, scale=scale).numpy().transpose(1, 0, 2)
        assert np.allclose(out[qs[b]:qs[b + 1]], ref, atol=1e-12, rtol=1e-12)


def test_single_query_is_decode():
    q, kc, vc, bt, cl, qs, scale = make(qlens=(1, 1, 1))
    out = oracle.decode_verify(q, kc, vc, bt, cl, qs, scale)
    assert np.allclose(out, oracle.decode_contiguous(q, kc, vc, bt, cl, scale), atol=1e-13)


def test_brute_force_and_last_row_is_full_decode():
    q, kc, vc, bt, cl, qs, scale = make(seed=1)
    out = oracle.decode_verify(q, kc, vc, bt, cl, qs, scale)
    BS = kc.shape[2]
    G = q.shape[1] // kc.shape[1]
    for b in range(len(cl)):
        L, q_b = int(cl[b]), int(qs[b + 1] - qs[b])
        for i in range(q_b):
            r = qs[b] + i
            for h in range(q.shape[1]):
                s, vs = [], []
                for t in range(L - q_b + i + 1):
                    pb, off = bt[b, t // BS], t % BS
                    s.append(scale * float(np.dot(q[r, h], kc[pb, h // G, off])))
                    vs.append(vc[pb, h // G, off])
                p = np.exp(np.array(s) - max(s))
                p /= p.sum()
                assert np.allclose(out[r, h], p @ np.array(vs), atol=1e-12)
        last = qs[b + 1] - 1
        full = oracle.decode_contiguous(q[last:last + 1], kc, vc, bt[b:b + 1], cl[b:b + 1], scale)
        assert np.allclose(out[last], full[0], atol=1e-13)


def test_causality():
    q, kc, vc, bt, cl, qs, scale = make(seed=2)
    base = oracle.decode_verify(q, kc, vc, bt, cl, qs, scale)
    BS = kc.shape[2]
    b, L, q_b = 2, int(cl[2]), int(qs[3] - qs[2])
    pos = L - q_b + 1                     # position of query row 1 of sequence 2
    kc2, vc2 = kc.copy(), vc.copy()
    for t in range(pos + 1, L):           # the future of row 1
        kc2[bt[b, t // BS], :, t % BS] += 3.0
        vc2[bt[b, t // BS], :, t % BS] -= 2.0
    out = oracle.decode_verify(q, kc2, vc2, bt, cl, qs, scale)
    assert np.array_equal(out[qs[2] + 1], base[qs[2] + 1])       # row 1 unchanged
    assert np.array_equal(out[qs[2]], base[qs[2]])               # row 0 unchanged
    assert not np.allclose(out[qs[2] + 2], base[qs[2] + 2])      # row 2 sees the change
    kc3 = kc.copy()
    kc3[bt[b, pos // BS], :, pos % BS] += 3.0                    # row 1's own token
    assert not np.allclose(oracle.decode_verify(q, kc3, vc, bt, cl, qs, scale)[qs[2] + 1],
                           base[qs[2] + 1])


def test_query_outside_history_gives_nan_rows():
    q, kc, vc, bt, cl, qs, scale = make(lens=(2, 5, 12), qlens=(3, 1, 4))
    out = oracle.decode_verify(q, kc, vc, bt, cl, qs, scale)
    assert np.isnan(out[0:3]).all() and np.isfinite(out[3:]).all()


# ---- planted mistakes: each must fail at least one pin above ----

def _verify_with(length_of):
    def f(query, key_cache, value_cache, block_tables, context_lens, query_start, scale):
        total_q, H, D = query.shape
        out = np.full((total_q, H, D), np.nan)
        qs = np.asarray(query_start, dtype=np.int64)
        for b in range(len(qs) - 1):
            q_b, L = int(qs[b + 1] - qs[b]), int(context_lens[b])
            if q_b <= 0 or q_b > L:
                continue
            for i in range(q_b):
                r = int(qs[b]) + i
                out[r] = oracle.decode_contiguous(query[r:r + 1], key_cache, value_cache,
                                                  np.asarray(block_tables)[b:b + 1],
                                                  np.array([length_of(L, q_b, i)]), scale)[0]
        return out
    return f


MUTANTS = {
    "off_by_one": _verify_with(lambda L, q, i: max(L - q + i, 1)),
    "not_causal": _verify_with(lambda L, q, i: L),
    "reversed_rows": _verify_with(lambda L, q, i: L - i),
}


def test_mutants_are_caught(monkeypatch):
    pins = [test_sdpa_with_causal_mask, test_single_query_is_decode,
            test_brute_force_and_last_row_is_full_decode, test_causality]
    for name, fn in MUTANTS.items():
        monkeypatch.setattr(oracle, "decode_verify", fn)
        caught = 0
        for pin in pins:
            try:
                pin()
            except AssertionError:
                caught += 1
        assert caught > 0, name
