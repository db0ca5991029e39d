"""Block and byte accounting against the pages' printed numbers (CPU only).

Fixture: tests/golden/worked_memory_example.json, from "What problem does
PagedAttention solve, and what is continuous batching?" (datarekha), section
"A concrete memory example" (formula and four-request table) and section
"How PagedAttention works" (the 50-token, 16-token-block example).
"""
import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import accounting as acc

MIB = 1 << 20


@pytest.fixture(scope="module")
def ex():
    return json.load(open(os.path.join(GOLDEN, "worked_memory_example.json")))


def test_bytes_per_token(ex):
    m = ex["model"]
    bpt = acc.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    assert bpt == ex["bytes_per_token"] == ex["bytes_per_token_kib"] * 1024


def test_request_table(ex):
    m, bs = ex["model"], ex["block_size"]
    bpt = acc.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    tot_tokens = tot_blocks = tot_alloc = 0
    for r in ex["requests"]:
        assert acc.blocks_needed(r["live_tokens"], bs) == r["blocks"]
        assert acc.allocated_bytes(r["live_tokens"], bs, bpt) == r["allocated_mib"] * MIB
        tot_tokens += r["live_tokens"]
        tot_blocks += r["blocks"]
        tot_alloc += acc.allocated_bytes(r["live_tokens"], bs, bpt)
    assert tot_tokens == ex["total"]["live_tokens"]
    assert tot_blocks == ex["total"]["blocks"]
    assert tot_alloc == ex["total"]["allocated_mib"] * MIB


def test_live_and_tail(ex):
    m, bs = ex["model"], ex["block_size"]
    bpt = acc.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    live = sum(acc.live_bytes(r["live_tokens"], bpt) for r in ex["requests"])
    tail = sum(acc.tail_bytes(r["live_tokens"], bs, bpt) for r in ex["requests"])
    assert live == ex["live_mib_approx"] * MIB        # exact: 6490 x 128 KiB
    assert tail == ex["tail_mib"] * MIB                # 38 tail tokens x 128 KiB
    assert sum(acc.tail_tokens(r["live_tokens"], bs) for r in ex["requests"]) == 38


def test_contiguous_reservation(ex):
    m = ex["model"]
    bpt = acc.kv_bytes_per_token(m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    per = acc.contiguous_reservation_bytes(ex["contiguous_reservation_tokens"], bpt)
    assert per == ex["contiguous_reservation_mib_per_request"] * MIB
    assert 4 * per == ex["contiguous_reservation_gib_for_four"] * (1 << 30)


def test_request_b_returns_its_blocks(ex):
    b = [r for r in ex["requests"] if r["name"] == "B"][0]
    assert acc.blocks_needed(b["live_tokens"], ex["block_size"]) == \
        ex["blocks_returned_when_B_finishes"]


def test_fifty_tokens_four_blocks():
    ex = json.load(open(os.path.join(GOLDEN, "block_table_example.json")))
    assert acc.blocks_needed(ex["num_tokens"], ex["block_size"]) == ex["logical_blocks"]
    assert acc.last_block_fill(ex["num_tokens"], ex["block_size"]) == ex["last_block_tokens"]
    assert ex["num_tokens"] // ex["block_size"] == ex["full_blocks"]


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_tail_is_under_one_block(bs):
    """Waste of a request is under one block: 0 <= alloc - live < bs tokens."""
    for L in range(0, 5 * bs + 1):
        t = acc.tail_tokens(L, bs)
        assert 0 <= t < bs
        assert acc.blocks_needed(L, bs) * bs - L == t


def test_effective_kv_bytes_of_worked_example(ex):
    """One layer of the worked example reads 6490 x 2 x 8 x 128 x 2 bytes."""
    lens = [r["live_tokens"] for r in ex["requests"]]
    assert acc.effective_kv_bytes(lens, 8, 128, 2) == 26_583_040
    assert 32 * acc.effective_kv_bytes(lens, 8, 128, 2) == ex["live_mib_approx"] * MIB
