"""Plant plausible mistakes in the block-pool oracle (on the CPU) and check
that the pins catch each one."""

import pytest

import test_block_pool_oracle as pins
from oracle import block_pool as bp


class NoCopyOnWrite(bp.BlockPool):
    """Writes into a shared partial block instead of copying it."""
    def append(self, table, token):
        table = list(table)
        if not table or len(self.tokens[table[-1]]) == self.block_size:
            table.append(self._take())
        last = table[-1]
        slot = last * self.block_size + len(self.tokens[last])
        self.tokens[last].append(token)
        return table, slot, None


class CopyWithoutData(bp.BlockPool):
    """Takes a fresh block on copy-on-write but does not copy the tokens."""
    def _take(self, initial=()):
        return super()._take(())


class CopyKeepsReference(bp.BlockPool):
    """Does not drop the branch's reference to the shared block."""
    def append(self, table, token):
        shared = bool(table) and len(self.tokens[table[-1]]) < self.block_size and \
            self.refs[table[-1]] > 1
        src = table[-1] if shared else None
        out = super().append(table, token)
        if shared:
            self.refs[src] += 1
        return out


class ForkWithoutReferences(bp.BlockPool):
    def fork(self, table):
        return list(table)


class FrontOfFreeList(bp.BlockPool):
    """Takes blocks from the front of the free list."""
    def _take(self, initial=()):
        if not self.free:
            raise bp.PoolExhausted("KV pool exhausted")
        b = self.free.pop(0)
        self.tokens[b] = list(initial)
        self.refs[b] = 1
        return b


class ReleaseFreesShared(bp.BlockPool):
    """Frees every block of a released table, shared or not."""
    def release(self, table):
        for b in table:
            self.refs[b] = 1
            self._drop(b)


class SlotOffByOne(bp.BlockPool):
    def append(self, table, token):
        t, slot, copy = super().append(table, token)
        return t, slot + 1, copy


MUTANTS = [NoCopyOnWrite, CopyWithoutData, CopyKeepsReference, ForkWithoutReferences,
           FrontOfFreeList, ReleaseFreesShared, SlotOffByOne]


def _pins_fail(monkeypatch, cls):
    monkeypatch.setattr(pins, "BlockPool", cls)
    failures = 0
    for pin in [pins.test_printed_cow_example] + \
               [lambda s=s: pins.test_random_operation_sequences(s) for s in range(6)]:
        try:
            pin()
        except Exception:
            failures += 1
    return failures


@pytest.mark.parametrize("cls", MUTANTS, ids=lambda c: c.__name__)
def test_mutant_is_caught(monkeypatch, cls):
    assert _pins_fail(monkeypatch, cls) > 0, cls.__name__


def test_unmutated_pool_passes(monkeypatch):
    assert _pins_fail(monkeypatch, bp.BlockPool) == 0
