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


def compare(lib_pool, ref, ids):
    for r, l in ids.items():
        assert list(lib_pool.table(l)) == ref.table(r)
        assert lib_pool.length(l) == ref.length(r)
    for b in range(ref.num_blocks):
        assert lib_pool.refcount(b) == ref.refcount(b)
    assert lib_pool.free_blocks() == len(ref.free)


@pytest.mark.parametrize("seed", range(25))
def test_random_operations_match_the_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    bs = int(rng.choice([1, 2, 3, 16, 32]))
    nb = int(rng.integers(4, 80))
    ref = oracle.BlockPool(nb, bs)
    lib_pool = ops.BlockPool(nb, bs)
    ids = {}                      # oracle sequence id -> library sequence id
    tok = 0
    for step in range(200):
        op = rng.choice(["new", "append", "append", "fork", "release"])
        if op == "new" or not ids:
            ids[ref.add_sequence()] = lib_pool.add_sequence()
        elif op == "append":
            live = list(ids)
            batch = [int(r) for r in rng.choice(live, size=int(rng.integers(1, len(live) + 1)),
                                                replace=False)]
            try:
                want_slots, want_pairs = ref.append(batch, list(range(tok, tok + len(batch))))
            except oracle.PoolExhausted:
                with pytest.raises(RuntimeError, match="exhausted"):
                    lib_pool.append([ids[r] for r in batch])
            else:
                slots, pairs = lib_pool.append([ids[r] for r in batch])
                assert slots.tolist() == want_slots
                assert pairs.tolist() == [list(p) for p in want_pairs]
                tok += len(batch)
        elif op == "fork":
            r = int(rng.choice(list(ids)))
            ids[ref.fork(r)] = lib_pool.fork(ids[r])
        else:
            r = int(rng.choice(list(ids)))
            ref.release(r)
            lib_pool.release(ids.pop(r))
        compare(lib_pool, ref, ids)
    for r in list(ids):
        lib_pool.release(ids.pop(r))
        ref.release(r)
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
