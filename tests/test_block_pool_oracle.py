"""Pins of the block-pool oracle: the worked example the page prints, and
invariants that must hold after any sequence of operations -- among them a
simulated device cache that makes every reported copy and slot write and
must then read back each sequence's history through its table."""

import json
import os

import numpy as np
import pytest

from oracle.block_pool import BlockPool, PoolExhausted, copy_blocks

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "block_pool_cow.json")


def test_printed_cow_example():
    g = json.load(open(GOLDEN))
    pool = BlockPool(g["num_blocks"], g["block_size"])
    orig = pool.add_sequence()
    for t in g["original_tokens"]:
        pool.append([orig], [t])
    branch = pool.fork(orig)
    slots, copies = pool.append([branch], [g["branch_append"]])
    a = g["asserted"]
    t_o, t_b = pool.table(orig), pool.table(branch)
    assert pool.read(orig) == a["read_original"]
    assert pool.read(branch) == a["read_branch"]
    assert (t_o[-1] != t_b[-1]) == a["tails_differ"]
    assert pool.refcount(t_o[0]) == a["refs_original_first"]
    assert pool.refcount(t_o[-1]) == a["refs_original_last"]
    d = g["derived"]
    assert t_o == d["original_table"] and t_b == d["branch_table"]
    assert copies == [tuple(d["copy"])]
    assert slots == [t_b[-1] * g["block_size"] + 1]


class DeviceCache:
    """What the device holds: one cell per slot, changed only by the copies
    and slot writes the pool reports, in the order a caller makes them."""

    def __init__(self, num_blocks, block_size):
        self.bs = block_size
        self.cells = np.full(num_blocks * block_size, -1, dtype=np.int64)

    def apply(self, slots, copies, tokens):
        bs = self.bs
        for src, dst in copies:
            self.cells[dst * bs:(dst + 1) * bs] = self.cells[src * bs:(src + 1) * bs]
        for s, tok in zip(slots, tokens):
            self.cells[s] = tok

    def read(self, table, length):
        return [int(self.cells[table[p // self.bs] * self.bs + p % self.bs]) for p in range(length)]


def check_invariants(pool, expect, cache):
    bs = pool.block_size
    assert set(pool.tables) == set(expect)
    named = {}
    for s, want in expect.items():
        t = pool.table(s)
        assert pool.read(s) == want and pool.length(s) == len(want)
        # a table names exactly the blocks its tokens need, each once
        assert len(t) == -(-len(want) // bs) and len(set(t)) == len(t)
        # the device cells the table points at hold the sequence's history
        assert cache.read(t, len(want)) == want
        for j, b in enumerate(t):
            named[b] = named.get(b, 0) + 1
            assert pool.contents(b)[:len(want[j * bs:(j + 1) * bs])] == want[j * bs:(j + 1) * bs]
    # every block is either free or named by a table, never both, and its
    # reference count is the number of tables naming it
    assert sorted(pool.free + list(named)) == list(range(pool.num_blocks))
    assert all(pool.refcount(b) == n for b, n in named.items())
    assert all(pool.refcount(b) == 0 for b in pool.free)


def snapshot(pool):
    return (list(pool.free), {s: pool.table(s) for s in pool.tables},
            {s: pool.read(s) for s in pool.history})


@pytest.mark.parametrize("seed", range(20))
def test_random_operation_sequences(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 2, 3, 16]))
    pool = BlockPool(int(rng.integers(8, 64)), bs)
    cache = DeviceCache(pool.num_blocks, bs)
    expect = {}
    next_tok = 1000
    for step in range(300):
        op = rng.choice(["new", "append", "append", "append", "fork", "release"])
        if op == "new" or not expect:
            expect[pool.add_sequence()] = []
        elif op == "append":
            live = list(expect)
            batch = [int(s) for s in rng.choice(live, size=int(rng.integers(1, len(live) + 1)),
                                                replace=False)]
            toks = list(range(next_tok, next_tok + len(batch)))
            before = snapshot(pool)
            try:
                slots, copies = pool.append(batch, toks)
            except PoolExhausted:
                assert snapshot(pool) == before          # all or nothing
                victim = int(rng.choice(live))
                pool.release(victim)
                expect.pop(victim)
            else:
                # each token lands in the block and offset its position names,
                # in a block no other table names; copies go to fresh blocks
                for s, slot in zip(batch, slots):
                    p = len(expect[s])
                    t = pool.table(s)
                    assert slot == t[p // bs] * bs + p % bs
                    assert pool.refcount(t[p // bs]) == 1
                for src, dst in copies:
                    assert dst in before[0] and src not in before[0]
                cache.apply(slots, copies, toks)
                for s, tok in zip(batch, toks):
                    expect[s] = expect[s] + [tok]
                next_tok += len(batch)
        elif op == "fork":
            s = int(rng.choice(list(expect)))
            expect[pool.fork(s)] = list(expect[s])
        else:
            s = int(rng.choice(list(expect)))
            pool.release(s)
            expect.pop(s)
        check_invariants(pool, expect, cache)
    for s in list(expect):
        pool.release(s)
    assert sorted(pool.free) == list(range(pool.num_blocks))
    assert all(pool.refcount(b) == 0 for b in range(pool.num_blocks))


def test_exhausted_pool_raises_and_changes_nothing():
    pool = BlockPool(2, 2)
    a = pool.add_sequence()
    for tok in (1, 2, 3, 4):
        pool.append([a], [tok])
    with pytest.raises(PoolExhausted):
        pool.append([a], [5])
    assert pool.read(a) == [1, 2, 3, 4] and pool.free == []


def test_three_holders_of_a_partial_block():
    # three sequences end in one partial block and all append: the first two
    # copy it, the last writes in place; with two holders of three listed,
    # both copy
    pool = BlockPool(8, 4)
    a = pool.add_sequence()
    pool.append([a], [1])
    b, c = pool.fork(a), pool.fork(a)
    shared = pool.table(a)[0]
    slots, copies = pool.append([b, a, c], [2, 3, 4])
    assert [src for src, _ in copies] == [shared, shared]
    assert pool.table(c) == [shared] and slots[2] == shared * 4 + 1
    pool2 = BlockPool(8, 4)
    a = pool2.add_sequence()
    pool2.append([a], [1])
    b, c = pool2.fork(a), pool2.fork(a)
    _, copies = pool2.append([a, b], [2, 3])
    assert len(copies) == 2 and pool2.refcount(pool2.table(c)[0]) == 1


def test_full_shared_tail_is_not_copied():
    # a full last block stays shared: the next token opens a fresh block
    pool = BlockPool(8, 2)
    a = pool.add_sequence()
    pool.append([a], [1])
    pool.append([a], [2])
    b = pool.fork(a)
    _, copies = pool.append([b], [3])
    assert copies == [] and pool.table(b)[0] == pool.table(a)[0]
    assert pool.refcount(pool.table(a)[0]) == 2


def test_copy_blocks_oracle():
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 2**16, size=(6, 2, 4, 8), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(6, 2, 4, 8), dtype=np.uint16)
    k2, v2 = copy_blocks(kc, vc, [(1, 4), (1, 5), (3, 0)])
    for src, dst in ((1, 4), (1, 5), (3, 0)):
        assert np.array_equal(k2[dst], kc[src]) and np.array_equal(v2[dst], vc[src])
    for b in (1, 2, 3):
        assert np.array_equal(k2[b], kc[b]) and np.array_equal(v2[b], vc[b])
