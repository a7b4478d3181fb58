"""Oracle of the shared, copy-on-write block pool and of the block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Rules, as the pages state them in prose ([vLLM-paging] "Copy-on-write 是共享的
正确性边界"; [MiniPaged-Qwen] §9 "差异 3" and §10.1 name the same features --
shared prefixes, branch sharing, reference counting, copy-on-write):

* a sequence owns a block table; token p of its history lives in block
  table[p // block_size] at offset p % block_size ([MiniPaged-Qwen] §6.2);
* a block's reference count is the number of live tables that name it, and
  a block no table names is free;
* forking a sequence gives the new sequence the same history and a table
  naming the same blocks (the blocks gain a reference each);
* a sequence may write only into a block no other table names: appending
  token p at offset 0 needs a fresh block; at a non-zero offset the block
  already exists, and if another table names it too, the sequence first
  takes a fresh block holding a copy of the shared one (the copy the device
  must make) and writes there;
* releasing a sequence drops its table.

The model is declarative: the state is each live sequence's token list and
table, plus the order of the free blocks.  Reference counts and block
contents are derived from them whenever asked (a block holds, slot by slot,
the tokens of any sequence naming it; sequences sharing a block agree on
it).  Fresh blocks come from the end of the free list and freed blocks go to
its end, in table order -- the allocation order of the pages' simulation,
under which its printed example names the blocks it does.

A batch of appends is taken in list order, each seeing the tables as the
earlier ones left them (of sequences sharing a partial block, every writer
but the last copies it); a batch that cannot get all its fresh blocks
changes nothing.

Each token's slot is block * block_size + offset, the linear slot the cache
write takes ([MiniPaged-Qwen] §8.1).

Parity status: pinned by the worked example of the page's simulation
(tests/golden/block_pool_cow.json) and by invariants under random operation
sequences, among them a simulated device cache that applies every copy and
slot write and must read back every sequence's history
(tests/test_block_pool_oracle.py).
"""

import numpy as np


class PoolExhausted(Exception):
    """No free block is left for an append (the simulation raises MemoryError)."""


class BlockPool:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks))   # fresh blocks come from the end
        self.history = {}                     # sequence id -> list of tokens
        self.tables = {}                      # sequence id -> list of blocks
        self._next = 0

    # -- derived quantities ---------------------------------------------
    def refcount(self, block):
        """Number of live tables naming the block."""
        return sum(t.count(block) for t in self.tables.values())

    def contents(self, block):
        """Tokens the block holds, read from a sequence that names it."""
        for s, t in self.tables.items():
            if block in t:
                j = t.index(block)
                return self.history[s][j * self.block_size:(j + 1) * self.block_size]
        return []

    def read(self, seq):
        return list(self.history[seq])

    def length(self, seq):
        return len(self.history[seq])

    def table(self, seq):
        return list(self.tables[seq])

    # -- operations -----------------------------------------------------
    def add_sequence(self):
        s = self._next
        self._next += 1
        self.history[s] = []
        self.tables[s] = []
        return s

    def fork(self, seq):
        s = self.add_sequence()
        self.history[s] = list(self.history[seq])
        self.tables[s] = list(self.tables[seq])
        return s

    def append(self, seqs, tokens):
        """Append tokens[i] to sequence seqs[i], in list order.  Returns
        (slots, copies): the slot of each token, and the (src, dst) block
        copies to make first, in order.  Raises PoolExhausted, changing
        nothing, when the fresh blocks do not suffice."""
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence is listed twice")
        tables = {s: list(t) for s, t in self.tables.items()}
        free = list(self.free)
        slots, copies = [], []
        for s, tok in zip(seqs, tokens):
            p = len(self.history[s])
            j, off = divmod(p, self.block_size)
            t = tables[s]
            if off == 0:
                if not free:
                    raise PoolExhausted("KV pool exhausted")
                t.append(free.pop())
            elif sum(u.count(t[j]) for u in tables.values()) > 1:
                if not free:
                    raise PoolExhausted("KV pool exhausted")
                fresh = free.pop()
                copies.append((t[j], fresh))
                t[j] = fresh
            slots.append(t[j] * self.block_size + off)
        # every append fits: commit
        self.tables, self.free = tables, free
        for s, tok in zip(seqs, tokens):
            self.history[s].append(tok)
        return slots, copies

    def release(self, seq):
        t = self.tables.pop(seq)
        del self.history[seq]
        for b in t:
            if self.refcount(b) == 0:
                self.free.append(b)


def copy_blocks(key_cache, value_cache, pairs):
    """key_cache[dst] = key_cache[src] (every KV head and slot of the block),
    the same for value_cache, for each (src, dst) in order: the physical
    copy behind a copy-on-write.  Works on raw bits of any dtype."""
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    for src, dst in pairs:
        kc[dst] = kc[src]
        vc[dst] = vc[src]
    return kc, vc
