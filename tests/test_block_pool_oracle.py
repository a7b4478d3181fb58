"""Pins of the block-pool oracle: the worked example the page prints, and
invariants that must hold after any sequence of operations."""

import json
import os

import numpy as np
import pytest

from oracle.block_pool import BlockPool, PoolExhausted, copy_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_pool_cow.json")


def test_printed_cow_example():
    g = json.load(open(GOLDEN))
    pool = BlockPool(g["num_blocks"], g["block_size"])
    orig = []
    for t in g["original_tokens"]:
        orig, _, _ = pool.append(orig, t)
    branch = pool.fork(orig)
    branch, slot, copy = pool.append(branch, g["branch_append"])
    a = g["asserted"]
    assert pool.read(orig) == a["read_original"]
    assert pool.read(branch) == a["read_branch"]
    assert (orig[-1] != branch[-1]) == a["tails_differ"]
    assert pool.refs[orig[0]] == a["refs_original_first"]
    assert pool.refs[orig[-1]] == a["refs_original_last"]
    d = g["derived"]
    assert orig == d["original_table"] and branch == d["branch_table"]
    assert copy == tuple(d["copy"])
    assert slot == branch[-1] * g["block_size"] + 1


def check_invariants(pool, tables, expect):
    # every block is either free or named by a table, never both; the
    # reference count is the number of tables naming the block
    named = {}
    for t in tables.values():
        for b in t:
            named[b] = named.get(b, 0) + 1
    assert named == pool.refs
    assert sorted(pool.free + list(named)) == list(range(pool.num_blocks))
    assert len(set(pool.free)) == len(pool.free)
    for k, t in tables.items():
        assert pool.read(t) == expect[k]
        # all blocks but the last are full; no empty block is held
        fills = [len(pool.tokens[b]) for b in t]
        assert all(f == pool.block_size for f in fills[:-1])
        assert all(f >= 1 for f in fills)
    # a block held by several tables is never written after the fork, so
    # every holder sees the same prefix of tokens there
    for b, n in pool.refs.items():
        if n > 1:
            assert len(pool.tokens[b]) <= pool.block_size


@pytest.mark.parametrize("seed", range(20))
def test_random_operation_sequences(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 3, 16]))
    pool = BlockPool(int(rng.integers(8, 64)), bs)
    tables, expect = {}, {}
    next_id, next_tok = 0, 1000
    for step in range(300):
        op = rng.choice(["new", "append", "append", "append", "fork", "release"])
        try:
            if op == "new" or not tables:
                tables[next_id], expect[next_id] = [], []
                next_id += 1
            elif op == "append":
                k = int(rng.choice(list(tables)))
                before = {b: list(pool.tokens[b]) for b in pool.tokens}
                t, slot, copy = pool.append(tables[k], next_tok)
                # the token lands in the slot the table's last block names
                assert slot // bs == t[-1] and slot % bs == len(expect[k]) % bs
                if copy is not None:
                    src, dst = copy
                    assert before[src] == pool.tokens[dst][:-1]   # copy of the shared block
                    assert pool.tokens[src] == before[src]        # the shared block is untouched
                tables[k] = t
                expect[k] = expect[k] + [next_tok]
                next_tok += 1
            elif op == "fork":
                k = int(rng.choice(list(tables)))
                tables[next_id] = pool.fork(tables[k])
                expect[next_id] = list(expect[k])
                next_id += 1
            else:
                k = int(rng.choice(list(tables)))
                pool.release(tables.pop(k))
                expect.pop(k)
        except PoolExhausted:
            k = int(rng.choice(list(tables)))
            pool.release(tables.pop(k))
            expect.pop(k)
        check_invariants(pool, tables, expect)
    for k in list(tables):
        pool.release(tables.pop(k))
    assert sorted(pool.free) == list(range(pool.num_blocks)) and not pool.refs


def test_exhausted_pool_raises_and_changes_nothing():
    pool = BlockPool(2, 2)
    t, _, _ = pool.append([], 1)
    t, _, _ = pool.append(t, 2)
    t, _, _ = pool.append(t, 3)          # second block
    t, _, _ = pool.append(t, 4)
    with pytest.raises(PoolExhausted):
        pool.append(t, 5)
    assert pool.read(t) == [1, 2, 3, 4] and pool.free == []


def test_full_shared_tail_is_not_copied():
    # a full last block stays shared: the next token opens a fresh block
    pool = BlockPool(8, 2)
    a, _, _ = pool.append([], 1)
    a, _, _ = pool.append(a, 2)
    b = pool.fork(a)
    b, _, copy = pool.append(b, 3)
    assert copy is None and b[0] == a[0] and pool.refs[a[0]] == 2


def test_copy_blocks_oracle():
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 2**16, size=(6, 2, 4, 8), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(6, 2, 4, 8), dtype=np.uint16)
    k2, v2 = copy_blocks(kc, vc, [(1, 4), (1, 5), (3, 0)])
    for src, dst in ((1, 4), (1, 5), (3, 0)):
        assert np.array_equal(k2[dst], kc[src]) and np.array_equal(v2[dst], vc[src])
    for b in (1, 2, 3):
        assert np.array_equal(k2[b], kc[b]) and np.array_equal(v2[b], vc[b])
