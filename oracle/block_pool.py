"""Oracle of the shared, copy-on-write block pool and of the block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is modelled ([vLLM-paging] "Copy-on-write 是共享的正确性边界" and its
"最小分页与 COW 模拟" simulation; [MiniPaged-Qwen] §9 "差异 3" and §10.1
name the same features -- shared prefixes, branch sharing, reference
counting, copy-on-write):

* a pool of physical blocks with a free list; a block is taken from the end
  of the free list and starts with reference count 1;
* a sequence is a block table (a list of physical blocks) whose blocks hold
  its tokens in order, block_size per block, the last one possibly partial;
* forking a sequence gives a second table naming the same blocks, and every
  block named gains one reference;
* appending a token: if the table is empty or its last block is full, a
  fresh block is taken and the token is its first; if the last block is
  partial but shared (more than one reference), the sequence may not write
  into it -- it drops its reference, takes a fresh block holding a copy of
  the shared block's tokens, and writes the token there; otherwise the token
  goes into the last block in place;
* releasing a sequence drops one reference of each of its blocks; a block
  with no reference left returns to the free list.

Each token's slot is block * block_size + position in the block, the linear
slot the cache write takes ([MiniPaged-Qwen] §8.1).  Token values are
tracked per block, so ``read`` returns exactly what the blocks hold.

Parity status: pinned by the worked example of the simulation (golden file
tests/golden/block_pool_cow.json) and by invariants under random operation
sequences (tests/test_block_pool_oracle.py).
"""

import numpy as np


class PoolExhausted(Exception):
    """No free block is left (the simulation raises MemoryError)."""


class BlockPool:
    def __init__(self, num_blocks, block_size):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("pool sizes must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks))
        self.tokens = {}       # block -> list of token values it holds
        self.refs = {}         # block -> number of tables naming it

    # -- blocks --------------------------------------------------------
    def _take(self, initial=()):
        if not self.free:
            raise PoolExhausted("KV pool exhausted")
        b = self.free.pop()
        self.tokens[b] = list(initial)
        self.refs[b] = 1
        return b

    def _drop(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            del self.refs[b]
            del self.tokens[b]
            self.free.append(b)

    # -- sequences -------------------------------------------------------
    def fork(self, table):
        for b in table:
            self.refs[b] += 1
        return list(table)

    def append(self, table, token):
        """Returns (new table, slot of the token, copy) with copy = (src,
        dst) when a shared partial block was copied, else None."""
        table = list(table)
        copy = None
        if not table or len(self.tokens[table[-1]]) == self.block_size:
            table.append(self._take())
        elif self.refs[table[-1]] > 1:
            src = table[-1]
            dst = self._take(self.tokens[src])
            self.refs[src] -= 1            # still held by another table
            table[-1] = dst
            copy = (src, dst)
        last = table[-1]
        slot = last * self.block_size + len(self.tokens[last])
        self.tokens[last].append(token)
        return table, slot, copy

    def release(self, table):
        for b in table:
            self._drop(b)

    def read(self, table):
        out = []
        for b in table:
            out.extend(self.tokens[b])
        return out

    def length(self, table):
        return sum(len(self.tokens[b]) for b in table)


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
