"""Plant plausible mistakes in the block-pool oracle (on the CPU) and check
that the pins catch each one.  Each mutant is the oracle's source with one
edit, compiled into a module of its own."""

import inspect
import types

import pytest

import test_block_pool_oracle as pins
from oracle import block_pool as bp

MUTANTS = {
    # writes into a shared partial block instead of copying it
    "no_copy_on_write": ("elif sum(u.count(t[j]) for u in tables.values()) > 1:", "elif False:"),
    # copies a partial block even when no other table names it
    "copy_unshared": ("for u in tables.values()) > 1:", "for u in tables.values()) >= 1:"),
    # counts holders before the batch, so every writer of a shared block copies
    "stale_counts_in_batch": ("for u in tables.values()) > 1:", "for u in self.tables.values()) > 1:"),
    # takes the fresh block but does not report the copy
    "copy_not_reported": ("copies.append((t[j], fresh))", "pass"),
    # the fork shares the parent's history list instead of copying it
    "fork_aliases_history": ("self.history[s] = list(self.history[seq])",
                             "self.history[s] = self.history[seq]"),
    # the fork starts with an empty table
    "fork_without_blocks": ("self.tables[s] = list(self.tables[seq])", "self.tables[s] = []"),
    # takes fresh blocks from the front of the free list
    "front_of_free_list": ("free.pop()", "free.pop(0)"),
    # frees every block of a released table, shared or not
    "release_frees_shared": ("if self.refcount(b) == 0:", "if True:"),
    # never returns blocks to the free list
    "release_leaks": ("if self.refcount(b) == 0:", "if False:"),
    # the slot is one past the token's place
    "slot_off_by_one": ("slots.append(t[j] * self.block_size + off)",
                        "slots.append(t[j] * self.block_size + off + 1)"),
    # the slot uses the logical block index instead of the physical block
    "slot_logical_block": ("slots.append(t[j] * self.block_size + off)",
                           "slots.append(j * self.block_size + off)"),
    # a batch that runs out of blocks keeps the appends made before it ran out
    "partial_batch": ("tables = {s: list(t) for s, t in self.tables.items()}\n        free = list(self.free)",
                      "tables = self.tables\n        free = self.free"),
}


def mutant_module(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(bp)
    assert old in src, name
    mod = types.ModuleType("block_pool_" + name)
    exec(compile(src.replace(old, new), mod.__name__, "exec"), mod.__dict__)
    return mod


def _pins_fail(monkeypatch, mod):
    monkeypatch.setattr(pins, "BlockPool", mod.BlockPool)
    monkeypatch.setattr(pins, "PoolExhausted", mod.PoolExhausted)
    failures = 0
    for pin in [pins.test_printed_cow_example] + \
               [lambda s=s: pins.test_random_operation_sequences(s) for s in range(6)]:
        try:
            pin()
        except Exception:
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(monkeypatch, name):
    assert _pins_fail(monkeypatch, mutant_module(name)) > 0, name


def test_unmutated_pool_passes(monkeypatch):
    mod = types.ModuleType("block_pool_plain")
    exec(compile(inspect.getsource(bp), mod.__name__, "exec"), mod.__dict__)
    assert _pins_fail(monkeypatch, mod) == 0
