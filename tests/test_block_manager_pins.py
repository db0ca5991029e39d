"""Pins of the block-manager model (oracle/block_manager.py) to what the pages
state, independent of the C++ manager it checks:

  * "What problem does PagedAttention solve, and what is continuous
    batching?" (datarekha), section "A concrete memory example": requests of
    3900, 420, 2100 and 70 tokens in 16-token blocks take 244, 27, 132 and 5
    blocks (408 in all); when request B finishes its 27 blocks return to the
    pool at once;
  * same page, "How PagedAttention works": 50 tokens take four logical blocks
    (three full, one holding two tokens); physical blocks 12, 87, 301, 44 hold
    positions 0..49 in order; the allocator can take any free block; the
    partly filled last block wastes at most the rest of one block;
    candidates sharing a prefix reference the same blocks, and a diverging
    candidate gets a private copy of the changed block;
  * "PagedAttention & Continuous Batching" (ai-ml-animation-academy),
    "If you remember three things": shared prefixes are shared blocks, i.e.
    prefix caching; waste falls to under one block per sequence.
"""
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle.block_manager import BlockManagerModel, NoBlocks

BS = 16


def _tokens(n, seed):
    return np.random.default_rng(seed).integers(0, 1 << 30, n).tolist()


def test_worked_example_blocks_and_b_returning():
    ex = json.load(open(os.path.join(GOLDEN, "worked_memory_example.json")))
    lens = [r["live_tokens"] for r in ex["requests"]]
    blocks = [r["blocks"] for r in ex["requests"]]
    bm = BlockManagerModel(4096, BS, np.random.default_rng(0).permutation(4096))
    for i, L in enumerate(lens):
        n_cached, slots = bm.add_sequence(i, _tokens(L, 100 + i))
        assert n_cached == 0 and len(slots) == L
    assert [len(bm.table(i)) for i in range(4)] == blocks
    assert sum(blocks) == ex["total"]["blocks"] == 4096 - bm.num_free()
    free_before = bm.num_free()
    bm.free_sequence(1)  # request B finishes
    assert bm.num_free() - free_before == blocks[1] == ex["blocks_returned_when_B_finishes"]
    # tail waste: under one block per sequence
    for i in (0, 2, 3):
        assert 0 <= len(bm.table(i)) * BS - bm.length(i) < BS


def test_fifty_tokens_in_blocks_12_87_301_44():
    ex = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    phys = ex["physical_blocks"]
    order = phys + [b for b in range(512) if b not in phys]
    bm = BlockManagerModel(512, ex["block_size"], order)
    _, slots = bm.add_sequence(7, _tokens(ex["num_tokens"], 7))
    assert bm.table(7) == phys
    assert len(bm.table(7)) == ex["logical_blocks"]
    assert bm.length(7) - (ex["logical_blocks"] - 1) * ex["block_size"] == ex["last_block_tokens"]
    assert int(slots[ex["derived"]["position"]]) == ex["derived"]["slot"]
    # positions are in order through the table
    assert [int(s) for s in slots] == [phys[p // 16] * 16 + p % 16 for p in range(50)]


def test_any_free_block_serves():
    """The allocator takes whatever block is free: non-contiguous ids work."""
    order = np.random.default_rng(3).permutation(64)
    bm = BlockManagerModel(64, BS, order)
    bm.add_sequence(0, _tokens(100, 1))
    assert bm.table(0) == [int(x) for x in order[:7]]


def test_fork_shares_blocks_and_divergence_copies_one_block():
    bm = BlockManagerModel(64, BS)
    bm.add_sequence(0, _tokens(50, 2))  # 3 full blocks + 2 tokens
    free = bm.num_free()
    bm.fork(0, 1)                       # beam candidate: same blocks, no copy
    assert bm.table(1) == bm.table(0) and bm.num_free() == free
    shared_last = bm.table(0)[-1]
    slots, cow = bm.append(1, [5])      # the candidate diverges
    assert len(cow) == 1 and cow[0][0] == shared_last
    private = cow[0][1]
    assert bm.table(1) == bm.table(0)[:-1] + [private]
    assert int(slots[0]) == private * BS + 2
    assert bm.num_free() == free - 1
    slots, cow = bm.append(0, [6])      # the parent's block is its own again
    assert cow == [] and int(slots[0]) == shared_last * BS + 2
    # full shared blocks are never copied: a new block is attached instead
    bm.append(0, [1] * 13)              # fills block 3 exactly (2 + 1 + 13 = 16)
    bm.fork(0, 2)
    slots, cow = bm.append(2, [9])
    assert cow == [] and bm.table(2)[:4] == bm.table(0)[:4] and len(bm.table(2)) == 5


def test_prefix_cache_reuses_full_blocks():
    bm = BlockManagerModel(1024, BS)
    prompt = _tokens(2048, 4)
    n, _ = bm.add_sequence(0, prompt)
    assert n == 0
    first = bm.table(0)
    n, slots = bm.add_sequence(1, prompt)      # the same system prompt
    assert n == 2048 and np.all(np.asarray(slots) == -1)
    assert bm.table(1) == first                 # shared blocks, nothing new
    # a prompt that agrees for 1000 tokens reuses 62 whole blocks
    other = prompt[:1000] + _tokens(500, 5)
    n, slots = bm.add_sequence(2, other)
    assert n == 62 * BS and bm.table(2)[:62] == first[:62]
    slots = np.asarray(slots)
    assert np.all(slots[:n] == -1) and np.all(slots[n:] >= 0)


def test_cached_blocks_survive_their_sequence_until_evicted():
    bm = BlockManagerModel(10, BS)
    prompt = _tokens(64, 6)                    # 4 full blocks
    bm.add_sequence(0, prompt)
    blocks = bm.table(0)
    bm.free_sequence(0)
    assert bm.num_free() == 10                 # cached blocks can be handed out
    n, _ = bm.add_sequence(1, prompt)          # ... but are found first
    assert n == 64 and bm.table(1) == blocks
    bm.free_sequence(1)
    # six fresh blocks come from the queue, then the oldest cached one goes
    bm.add_sequence(2, _tokens(16 * 7, 7))
    assert blocks[0] in bm.table(2)
    bm.free_sequence(2)
    n, _ = bm.add_sequence(3, prompt)          # its first block is gone
    assert n == 0


def test_no_blocks_changes_nothing():
    bm = BlockManagerModel(10, BS)
    bm.add_sequence(0, _tokens(16 * 9, 8))
    state = (bm.num_free(), bm.table(0))
    with pytest.raises(NoBlocks):
        bm.add_sequence(1, _tokens(33, 9))     # needs 3 blocks, 1 free
    with pytest.raises(NoBlocks):
        bm.append(0, _tokens(17, 10))          # needs 2 blocks
    assert (bm.num_free(), bm.table(0)) == state and 1 not in bm.seqs


def test_decode_step_parent_and_candidate_share_one_copy():
    """Both beam candidates append in one step: the first to write gets the
    private copy, after which the shared block is the other's alone."""
    bm = BlockManagerModel(16, BS)
    bm.add_sequence(0, _tokens(20, 11))    # one full block + 4 tokens
    bm.fork(0, 1)
    shared = bm.table(0)[-1]
    slots, cow = bm.append_batch([0, 1], [3, 4])
    assert len(cow) == 1 and cow[0][0] == shared
    assert bm.table(0)[-1] == cow[0][1] and bm.table(1)[-1] == shared
    assert slots == [cow[0][1] * BS + 4, shared * BS + 4]


def test_decode_step_is_all_or_nothing():
    bm = BlockManagerModel(4, BS)
    for s in range(3):
        bm.add_sequence(s, _tokens(16, 20 + s))   # three full blocks, one free
    state = (bm.num_free(), [bm.table(s) for s in range(3)], [bm.length(s) for s in range(3)])
    with pytest.raises(NoBlocks):
        bm.append_batch([0, 1, 2], [1, 2, 3])     # needs three new blocks
    assert (bm.num_free(), [bm.table(s) for s in range(3)],
            [bm.length(s) for s in range(3)]) == state
