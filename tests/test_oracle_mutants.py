"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin fails for each.  This is what makes the pins evidence: a
dropped term, a wrong sign, a wrong index or a transposed operand anywhere in
the oracle must be caught."""

import math

import numpy as np
import pytest

import oracle_pins
from oracle import paged_attention as pa


def _softmax_unnormalised(s):
    return np.exp(s - s.max())


def _softmax_no_max(s):
    e = np.exp(s)
    return e / e.sum()


def _softmax_sign(s):
    e = np.exp(s.max() - s)
    return e / e.sum()


def _gather_no_transpose(key_cache, value_cache, row, L, kv_heads=None):
    N, H_kv, BS, D = key_cache.shape
    kv_heads = list(range(H_kv)) if kv_heads is None else kv_heads
    T = pa.num_logical_blocks(L, BS)
    ids = np.asarray(row[:T], dtype=np.int64)
    kvh = np.asarray(kv_heads)
    K = key_cache[ids][:, kvh].reshape(len(kvh), T * BS, D)[:, :L]
    V = value_cache[ids][:, kvh].reshape(len(kvh), T * BS, D)[:, :L]
    return K, V


def _gather_drops_last(key_cache, value_cache, row, L, kv_heads=None):
    K, V = _ORIG["gather"](key_cache, value_cache, row, L, kv_heads)
    keep = max(L - 1, 1) if L > 0 else 0
    return K[:, :keep], V[:, :keep]


def _gather_reversed_table(key_cache, value_cache, row, L, kv_heads=None):
    T = pa.num_logical_blocks(L, key_cache.shape[2])
    rev = list(row[:T])[::-1]
    return _ORIG["gather"](key_cache, value_cache, rev, L, kv_heads)


def _walk_factory(variant):
    def walk(qv, key_cache, value_cache, row, kvh, t0, t1, scale):
        BS, D = key_cache.shape[2], key_cache.shape[3]
        m, l, acc = pa.NEG_INF, 0.0, np.zeros(D)
        if t1 <= t0:
            return m, l, acc
        for t in range(t0 // BS, (t1 - 1) // BS + 1):
            pb = int(row[t])
            lo = max(t0 - t * BS, 0)
            hi = min(t1 - t * BS, BS)
            if variant == "no_tail_mask":
                hi = BS if t1 - t * BS < BS and t1 - t * BS > 0 else hi
            Kt = key_cache[pb, kvh, lo:hi].astype(np.float64)
            Vt = value_cache[pb, kvh, lo:hi].astype(np.float64)
            s = float(scale) * (Kt @ qv)
            m_new = max(m, float(s.max()))
            if variant == "alpha_sign":
                alpha = 0.0 if m == pa.NEG_INF else math.exp(m_new - m)
            else:
                alpha = 0.0 if m == pa.NEG_INF else math.exp(m - m_new)
            if variant == "local_max":
                e = np.exp(s - float(s.max()))
            else:
                e = np.exp(s - m_new)
            if variant == "l_not_rescaled":
                l = l + float(e.sum())
            else:
                l = l * alpha + float(e.sum())
            if variant == "acc_not_rescaled":
                acc = acc + e @ Vt
            elif variant == "per_block_softmax":
                # the per-block normalisation of the PA-source §4 sketch
                acc = acc + (e / e.sum()) @ Vt
                l = 1.0
            else:
                acc = acc * alpha + e @ Vt
            m = m_new
        return m, l, acc
    return walk


def _merge_sign(lses, outs):
    lses = np.asarray(lses, dtype=np.float64)
    w = np.exp(lses.max() - lses)
    return sum(w[p] * outs[p] for p in range(len(lses))) / w.sum()


def _merge_unweighted(lses, outs):
    return sum(outs) / len(outs)


def _kv_head_interleaved(h, num_heads, num_kv_heads):
    return int(h) % int(num_kv_heads)


def _cache_write_transposed(key, value, key_cache, value_cache, slot_mapping):
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    BS = kc.shape[2]
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        kc[s % BS, :, s // BS, :] = key[i]
        vc[s % BS, :, s // BS, :] = value[i]
    return kc, vc


def _cache_write_off_by_one(key, value, key_cache, value_cache, slot_mapping):
    return _ORIG["write"](key, value, key_cache, value_cache,
                          [s + 1 if s >= 0 else s for s in slot_mapping])


def _ceil_floor(L, block_size):
    return int(L) // int(block_size)


_ORIG = {"gather": pa.gather_sequence_kv, "write": pa.reshape_and_cache}

MUTANTS = {
    "softmax_unnormalised": [("_softmax", _softmax_unnormalised)],
    "softmax_without_max": [("_softmax", _softmax_no_max)],
    "softmax_sign": [("_softmax", _softmax_sign)],
    "gather_no_transpose": [("gather_sequence_kv", _gather_no_transpose)],
    "gather_drops_last_token": [("gather_sequence_kv", _gather_drops_last)],
    "gather_reversed_table": [("gather_sequence_kv", _gather_reversed_table)],
    "walk_alpha_sign": [("_online_walk", _walk_factory("alpha_sign"))],
    "walk_local_max": [("_online_walk", _walk_factory("local_max"))],
    "walk_l_not_rescaled": [("_online_walk", _walk_factory("l_not_rescaled"))],
    "walk_acc_not_rescaled": [("_online_walk", _walk_factory("acc_not_rescaled"))],
    "walk_per_block_softmax": [("_online_walk", _walk_factory("per_block_softmax"))],
    "walk_no_tail_mask": [("_online_walk", _walk_factory("no_tail_mask"))],
    "merge_sign": [("lse_merge", _merge_sign)],
    "merge_unweighted": [("lse_merge", _merge_unweighted)],
    "kv_head_interleaved": [("kv_head_of", _kv_head_interleaved)],
    "cache_write_transposed": [("reshape_and_cache", _cache_write_transposed)],
    "cache_write_off_by_one": [("reshape_and_cache", _cache_write_off_by_one)],
    "block_count_floor": [("num_logical_blocks", _ceil_floor)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    import oracle
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(pa, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # AssertionError, or an index/shape error
            failed.append((pin.__name__, type(e).__name__))
            break
    assert failed, "planted mistake %r passed every pin" % name
