"""The host-side slot-mapping check (pa_check_slot_mapping) through the C ABI:
distinct in-pool slots pass, padding passes, a slot past the pool or a slot
given twice is rejected with the token(s) named.  Host memory only."""

import numpy as np
import pytest

from paged_kv_decode_attention_amd import ops


def test_distinct_slots_and_padding_pass():
    ops.check_slot_mapping(np.array([5, -1, 0, 7, -3, 2], dtype=np.int64), 8)
    ops.check_slot_mapping(np.zeros(0, dtype=np.int64), 0)
    ops.check_slot_mapping(np.full(4, -1, dtype=np.int64), 0)
    rng = np.random.default_rng(0)
    ops.check_slot_mapping(rng.permutation(100000)[:4096], 100000)


def test_duplicate_slot_is_named():
    with pytest.raises(RuntimeError, match="slot 7 given to tokens 1 and 4"):
        ops.check_slot_mapping(np.array([3, 7, -1, 9, 7], dtype=np.int64), 16)


def test_slot_past_the_pool_is_named():
    with pytest.raises(RuntimeError, match="token 2: slot 16 is past the pool"):
        ops.check_slot_mapping(np.array([0, 15, 16], dtype=np.int64), 16)


def test_pool_slots_pass_the_check():
    # the slots a batch append hands out are distinct by construction
    pool = ops.BlockPool(64, 4)
    seqs = [pool.add_sequence() for _ in range(5)]
    for _ in range(9):
        slots, _ = pool.append(seqs)
        ops.check_slot_mapping(slots, 64 * 4)
    seqs.append(pool.fork(seqs[0]))
    slots, _ = pool.append(seqs)
    ops.check_slot_mapping(slots, 64 * 4)


def test_bad_counts_rejected():
    lib = ops.load_library()
    assert lib.pa_check_slot_mapping(None, -1, 4) == -1     # PA_ERR_INVALID_ARG
    assert lib.pa_check_slot_mapping(None, 3, 4) == -1
