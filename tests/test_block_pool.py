"""The library's block pool (pa_pool_*, host code behind the C ABI) against
the block-pool oracle, operation by operation: tables, token slots, copy
pairs, reference counts and free lists must agree exactly."""

import json
import os

import numpy as np
import pytest

import oracle
from paged_kv_decode_attention_amd import ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_pool_cow.json")


def test_printed_cow_example_through_the_library():
    g = json.load(open(GOLDEN))
    pool = ops.BlockPool(g["num_blocks"], g["block_size"])
    orig = pool.add_sequence()
    for _ in g["original_tokens"]:
        pool.append([orig])
    branch = pool.fork(orig)
    slots, pairs = pool.append([branch])
    t_o, t_b = list(pool.table(orig)), list(pool.table(branch))
    assert t_o == g["derived"]["original_table"] and t_b == g["derived"]["branch_table"]
    assert pairs.tolist() == [g["derived"]["copy"]]
    assert (t_o[-1] != t_b[-1]) == g["asserted"]["tails_differ"]
    assert pool.refcount(t_o[0]) == g["asserted"]["refs_original_first"]
    assert pool.refcount(t_o[-1]) == g["asserted"]["refs_original_last"]
    assert pool.length(orig) == 3 and pool.length(branch) == 4
    assert slots.tolist() == [t_b[-1] * g["block_size"] + 1]


def compare(lib_pool, ref, tables, ids):
    for k, t in tables.items():
        assert list(lib_pool.table(ids[k])) == t
        assert lib_pool.length(ids[k]) == ref.length(t)
    for b in range(ref.num_blocks):
        assert lib_pool.refcount(b) == ref.refs.get(b, 0)
    assert lib_pool.free_blocks() == len(ref.free)


@pytest.mark.parametrize("seed", range(25))
def test_random_operations_match_the_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([1, 2, 3, 16, 32]))
    nb = int(rng.integers(4, 80))
    ref = oracle.BlockPool(nb, bs)
    lib_pool = ops.BlockPool(nb, bs)
    tables, ids = {}, {}          # key -> oracle table, key -> library id
    key, tok = 0, 0
    for step in range(200):
        op = rng.choice(["new", "append", "append", "fork", "release"])
        if op == "new" or not tables:
            tables[key], ids[key] = [], lib_pool.add_sequence()
            key += 1
        elif op == "append":
            keys = list(tables)
            batch = list(rng.choice(keys, size=int(rng.integers(1, len(keys) + 1)),
                                    replace=False))
            # the oracle, one append after another in list order
            trial = oracle.BlockPool(nb, bs)
            trial.free, trial.tokens, trial.refs = (list(ref.free),
                                                    {b: list(v) for b, v in ref.tokens.items()},
                                                    dict(ref.refs))
            want_slots, want_pairs, new_tables = [], [], {}
            try:
                for k in batch:
                    t, slot, copy = trial.append(new_tables.get(k, tables[k]), tok + len(want_slots))
                    new_tables[k] = t
                    want_slots.append(slot)
                    if copy is not None:
                        want_pairs.append(list(copy))
                exhausted = False
            except oracle.PoolExhausted:
                exhausted = True
            if exhausted:
                with pytest.raises(RuntimeError, match="exhausted"):
                    lib_pool.append([ids[k] for k in batch])
            else:
                slots, pairs = lib_pool.append([ids[k] for k in batch])
                assert slots.tolist() == want_slots
                assert pairs.tolist() == want_pairs
                ref = trial
                tables.update(new_tables)
                tok += len(batch)
        elif op == "fork":
            k = int(rng.choice(list(tables)))
            tables[key], ids[key] = ref.fork(tables[k]), lib_pool.fork(ids[k])
            key += 1
        else:
            k = int(rng.choice(list(tables)))
            ref.release(tables.pop(k))
            lib_pool.release(ids.pop(k))
        compare(lib_pool, ref, tables, ids)
    for k in list(tables):
        lib_pool.release(ids.pop(k))
        ref.release(tables.pop(k))
    assert lib_pool.free_blocks() == nb


def test_pool_errors():
    pool = ops.BlockPool(2, 4)
    a = pool.add_sequence()
    with pytest.raises(RuntimeError, match="listed twice"):
        pool.append([a, a])
    with pytest.raises(RuntimeError, match="unknown sequence"):
        pool.append([a + 7])
    pool.append([a])
    b = pool.fork(a)
    c = pool.fork(a)
    # three sequences on one partial block: two copies are needed, one free
    # block is left -> nothing may change
    with pytest.raises(RuntimeError, match="exhausted"):
        pool.append([a, b, c])
    assert pool.refcount(pool.table(a)[0]) == 3 and pool.free_blocks() == 1
    assert [pool.length(s) for s in (a, b, c)] == [1, 1, 1]
    pool.release(b)
    with pytest.raises(RuntimeError, match="unknown sequence"):
        pool.release(b)
    with pytest.raises(RuntimeError, match="unknown sequence"):
        pool.fork(b)
    lib = ops.load_library()
    assert not lib.pa_pool_create(0, 16)
    assert lib.pa_pool_refcount(pool._h, 99) == -1     # PA_ERR_INVALID_ARG
