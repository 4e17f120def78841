"""Pins for the oracle block manager against what the pages state: the Day 3
worked example, waste confined to the last block, sharing by reference and
copy only on write."""

import json
import os

import pytest

from oracle.block_manager import BlockManagerOracle, NoFreeBlock

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_blocks_and_last_block_fill():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_block_table.json")))
    bm = BlockManagerOracle(num_blocks=10, block_size=ex["block_size"])
    bm.add_sequence(0)
    for _ in range(ex["seq_len"]):
        bm.append_token(0)
    table = bm.tables[0]
    assert len(table) == len(ex["block_table"])             # 37 tokens -> 3 blocks
    held = [min(ex["block_size"], ex["seq_len"] - i * ex["block_size"]) for i in range(len(table))]
    assert held == sorted(ex["tokens_held"].values(), reverse=True)   # 16, 16, 5
    assert bm.lens[0] == 37 and len(bm.free) == 7


@pytest.mark.parametrize("n", [1, 15, 16, 17, 100, 257])
def test_new_block_only_when_the_last_is_full(n):
    bm = BlockManagerOracle(64, 16)
    bm.add_sequence(7)
    for t in range(n):
        before = len(bm.tables[7])
        block, off = bm.append_token(7)
        assert off == t % 16
        assert len(bm.tables[7]) == before + (1 if t % 16 == 0 else 0)
    assert len(bm.tables[7]) * 16 - n < 16                  # waste below one block


def test_fork_shares_and_copies_only_a_partial_last_block():
    bm = BlockManagerOracle(32, 16)
    bm.add_sequence(0)
    for _ in range(40):                                       # blocks 0, 1, 2 (8 tokens in 2)
        bm.append_token(0)
    bm.fork(0, 1)
    assert bm.tables[1] == bm.tables[0] and [bm.ref[b] for b in bm.tables[0]] == [2, 2, 2]
    assert bm.take_copies() == []
    b, off = bm.append_token(1)                               # writes into shared block 2
    assert off == 8 and b != 2
    assert bm.take_copies() == [(2, b)]
    assert bm.tables[1][:2] == bm.tables[0][:2] and bm.ref[2] == 1
    b0, _ = bm.append_token(0)                                # sole holder now: in place
    assert b0 == 2 and bm.take_copies() == []


def test_full_shared_block_needs_no_copy():
    bm = BlockManagerOracle(8, 16)
    bm.add_sequence(0)
    for _ in range(32):
        bm.append_token(0)
    bm.fork(0, 1)
    b, off = bm.append_token(1)
    assert off == 0 and b not in bm.tables[0] and bm.take_copies() == []


def test_eight_way_share_makes_seven_copies():
    bm = BlockManagerOracle(128, 16)
    bm.add_sequence(0)
    for _ in range(1032):                                     # 64 full blocks + 8 tokens
        bm.append_token(0)
    for s in range(1, 8):
        bm.fork(0, s)
    for s in range(8):
        bm.append_token(s)
    copies = bm.take_copies()
    assert len(copies) == 7 and {src for src, _ in copies} == {bm.tables[7][64]}
    assert all(bm.ref[b] == 8 for b in bm.tables[0][:64])


def test_free_returns_blocks_and_exhaustion_is_reported():
    bm = BlockManagerOracle(3, 4)
    bm.add_sequence(0)
    for _ in range(12):
        bm.append_token(0)
    with pytest.raises(NoFreeBlock):
        bm.append_token(0)
    bm.fork(0, 1)
    bm.free_sequence(0)
    assert bm.free == [] and all(r == 1 for r in bm.ref)
    bm.free_sequence(1)
    assert sorted(bm.free) == [0, 1, 2] and bm.free[-1] == 2  # last block on top
