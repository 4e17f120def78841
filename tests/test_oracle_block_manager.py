"""Pins for the oracle block manager against what the pages state: the Day 3
worked example, waste confined to the last block, sharing by reference and
copy only on write."""

import json
import random
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


# ------------------------------------------------------------------- swapping
# The pages (supersilo.blog summary, section "적용 범위와 관련 연구") say
# sequences move to CPU memory when device memory runs short and come back
# later. What must hold whatever the mechanism: the device blocks are given
# back, and after the way back every sequence reads exactly its history.

class Contents:
    """Token ids held by every slot of the device and host pools, moved by
    the planned copies in the order a step runs them (swap-out pairs, then
    swap-in pairs, then copy-on-write pairs, then the new tokens)."""

    def __init__(self, num_blocks, num_host_blocks, block_size):
        self.dev = [[None] * block_size for _ in range(num_blocks)]
        self.host = [[None] * block_size for _ in range(num_host_blocks)]
        self.bs = block_size

    def run_step(self, out_pairs=(), in_pairs=(), copies=(), writes=()):
        for d, h in out_pairs:
            self.host[h] = list(self.dev[d])
        for h, d in in_pairs:
            self.dev[d] = list(self.host[h])
        for s, d in copies:
            self.dev[d] = list(self.dev[s])
        for (block, off), tok in writes:
            self.dev[block][off] = tok

    def history(self, bm, seq):
        pool = self.host if seq in bm.swapped else self.dev
        return [pool[bm.tables[seq][t // self.bs]][t % self.bs] for t in range(bm.lens[seq])]


def _grow(bm, contents, seq, hist, n, next_tok):
    for _ in range(n):
        slot = bm.append_token(seq)
        contents.run_step(copies=bm.take_copies(), writes=[(slot, next_tok)])
        hist[seq].append(next_tok)
        next_tok += 1
    return next_tok


def test_swap_out_returns_device_blocks_and_swap_in_restores_the_history():
    bm = BlockManagerOracle(num_blocks=10, block_size=16, num_host_blocks=6)
    c, hist = Contents(10, 6, 16), {0: []}
    bm.add_sequence(0)
    _grow(bm, c, 0, hist, 37, 1000)                           # 3 blocks, the last holds 5
    dev_table = list(bm.tables[0])
    out = bm.swap_out([0])
    assert [d for d, _ in out] == dev_table and len(bm.free) == 10
    assert bm.host_ref == [1, 1, 1, 0, 0, 0] and len(bm.host_free) == 3
    c.run_step(out_pairs=out)
    assert c.history(bm, 0) == hist[0]
    # the device blocks are reused meanwhile
    bm.add_sequence(1)
    hist[1] = []
    _grow(bm, c, 1, hist, 40, 5000)
    back = bm.swap_in([0])
    assert [h for h, _ in back] == [h for _, h in out]
    assert not set(bm.tables[0]) & set(bm.tables[1])
    c.run_step(in_pairs=back)
    assert c.history(bm, 0) == hist[0] and c.history(bm, 1) == hist[1]
    assert len(bm.host_free) == 6 and bm.host_free[-1] == out[-1][1]   # last block on top
    _grow(bm, c, 0, hist, 20, 9000)                           # it grows again after the return
    assert c.history(bm, 0) == hist[0]


def test_shared_blocks_move_once_and_stay_shared():
    bm = BlockManagerOracle(num_blocks=200, block_size=16, num_host_blocks=80)
    c, hist = Contents(200, 80, 16), {0: []}
    bm.add_sequence(0)
    _grow(bm, c, 0, hist, 1032, 0)                            # 64 full blocks + 8 tokens
    for s in range(1, 8):
        bm.fork(0, s)
        hist[s] = list(hist[0])
    tok = 10000
    for s in range(8):                                        # 7 copies of the partial block
        tok = _grow(bm, c, s, hist, 1, tok)
    used = 200 - len(bm.free)
    out = bm.swap_out(list(range(8)))
    assert len(out) == used == 64 + 8 and len(bm.free) == 200
    assert all(bm.host_ref[bm.tables[0][i]] == 8 for i in range(64))
    c.run_step(out_pairs=out)
    back = bm.swap_in(list(range(8)))
    assert len(back) == 72 and all(bm.ref[bm.tables[0][i]] == 8 for i in range(64))
    c.run_step(in_pairs=back)
    for s in range(8):
        assert c.history(bm, s) == hist[s]


def test_swapping_part_of_a_group_leaves_the_rest_in_place():
    bm = BlockManagerOracle(num_blocks=20, block_size=4, num_host_blocks=20)
    c, hist = Contents(20, 20, 4), {0: []}
    bm.add_sequence(0)
    _grow(bm, c, 0, hist, 10, 0)                              # blocks 0, 1, 2 (2 tokens in 2)
    bm.fork(0, 1)
    hist[1] = list(hist[0])
    shared = list(bm.tables[0])
    out = bm.swap_out([1])
    assert [d for d, _ in out] == shared
    assert bm.tables[0] == shared and all(bm.ref[b] == 1 for b in shared) and len(bm.free) == 17
    c.run_step(out_pairs=out)
    _grow(bm, c, 0, hist, 3, 100)                             # sole holder again: in place
    assert bm.tables[0][:3] == shared
    back = bm.swap_in([1])
    c.run_step(in_pairs=back)
    assert c.history(bm, 0) == hist[0] and c.history(bm, 1) == hist[1]


def test_swap_is_all_or_nothing():
    bm = BlockManagerOracle(num_blocks=12, block_size=4, num_host_blocks=3)
    for s in (0, 1):
        bm.add_sequence(s)
        for _ in range(8):
            bm.append_token(s)
    before = (dict(bm.tables), list(bm.ref), list(bm.free), list(bm.host_ref), list(bm.host_free))
    with pytest.raises(NoFreeBlock):
        bm.swap_out([0, 1])                                   # 4 blocks, 3 host blocks
    assert (dict(bm.tables), list(bm.ref), list(bm.free), list(bm.host_ref),
            list(bm.host_free)) == before and not bm.swapped
    bm.swap_out([0])
    for _ in range(4):                                        # seq 1: 3 blocks
        bm.append_token(1)
    bm.add_sequence(2)
    for _ in range(36):                                       # seq 2: 9 blocks, none left
        bm.append_token(2)
    free_before = list(bm.free)
    with pytest.raises(NoFreeBlock):
        bm.swap_in([0])                                       # 2 blocks, 0 free
    assert bm.free == free_before and 0 in bm.swapped


def test_swapped_sequences_neither_grow_nor_fork_and_queued_copies_block_a_swap():
    bm = BlockManagerOracle(num_blocks=8, block_size=4, num_host_blocks=8)
    bm.add_sequence(0)
    for _ in range(6):
        bm.append_token(0)
    bm.fork(0, 1)
    bm.append_token(1)                                        # queues a copy
    with pytest.raises(AssertionError):
        bm.swap_out([0])
    bm.take_copies()
    bm.swap_out([0])
    for op in (lambda: bm.append_token(0), lambda: bm.fork(0, 2), lambda: bm.swap_out([0])):
        with pytest.raises(AssertionError):
            op()
    bm.free_sequence(0)
    assert len(bm.host_free) == 8 and 0 not in bm.swapped


@pytest.mark.parametrize("seed", range(4))
def test_random_steps_keep_every_history(seed):
    """Random steps of a scheduler: swap some sequences out, some back in,
    grow the resident ones (forks, frees, copy-on-write included); after each
    step every sequence reads its own history through its table."""
    rng = random.Random(seed)
    nb, nh, bs = 24, 24, 4
    bm, c = BlockManagerOracle(nb, bs, nh), Contents(nb, nh, bs)
    hist, tok, next_id = {}, 0, 0
    for _ in range(150):
        live = sorted(bm.tables)
        resident = [s for s in live if s not in bm.swapped]
        out = ins = []
        if resident and rng.random() < 0.25:
            pick = rng.sample(resident, rng.randint(1, len(resident)))
            try:
                out = bm.swap_out(pick)
            except NoFreeBlock:
                out = []
        swapped = sorted(bm.swapped)
        if swapped and rng.random() < 0.3:
            pick = rng.sample(swapped, rng.randint(1, len(swapped)))
            try:
                ins = bm.swap_in(pick)
            except NoFreeBlock:
                ins = []
        op = rng.random()
        if op < 0.15 or not live:
            bm.add_sequence(next_id)
            hist[next_id] = []
            next_id += 1
        elif op < 0.25 and resident:
            parent = rng.choice([s for s in resident if s in bm.tables and s not in bm.swapped]
                                or [None])
            if parent is not None:
                bm.fork(parent, next_id)
                hist[next_id] = list(hist[parent])
                next_id += 1
        elif op < 0.32:
            s = rng.choice(live)
            bm.free_sequence(s)
            del hist[s]
        writes = []
        for s in sorted(bm.tables):
            if s in bm.swapped or rng.random() < 0.4:
                continue
            try:
                writes.append((bm.append_token(s), tok))
            except NoFreeBlock:
                continue
            hist[s].append(tok)
            tok += 1
        c.run_step(out, ins, bm.take_copies(), writes)
        for s in bm.tables:
            assert c.history(bm, s) == hist[s]
        assert len(bm.free) + sum(1 for r in bm.ref if r) == nb
        assert len(bm.host_free) + sum(1 for r in bm.host_ref if r) == nh


# --------------------------------------------------------- shared prefixes
# Samples forked from one prompt read the prompt's blocks by reference
# ([summary] "블록 공유"); the grouped decode reads such blocks once per group.
# What must hold: inside the reported shared tokens, every sequence of the
# group holds the same token in the same place.

def test_shared_prefix_of_forked_samples():
    bm = BlockManagerOracle(num_blocks=200, block_size=16)
    c, hist = Contents(200, 0, 16), {0: []}
    bm.add_sequence(0)
    _grow(bm, c, 0, hist, 1032, 0)                            # 64 full blocks + 8 tokens
    for s in range(1, 8):
        bm.fork(0, s)
        hist[s] = list(hist[0])
    assert bm.shared_prefix(list(range(8)), 8) == [65 * 16]   # the partial block too, for now
    tok = 5000
    for s in range(8):
        tok = _grow(bm, c, s, hist, 1, tok)                   # copy-on-write of the partial block
    assert bm.shared_prefix(list(range(8)), 8) == [64 * 16]
    assert bm.shared_prefix(list(range(8)), 4) == [64 * 16, 64 * 16]
    assert bm.shared_prefix(list(range(8)), 1) == [len(bm.tables[s]) * 16 for s in range(8)]
    bm.add_sequence(99)
    for _ in range(40):
        bm.append_token(99)
    assert bm.shared_prefix([0, 99], 2) == [0]


@pytest.mark.parametrize("seed", range(4))
def test_shared_tokens_hold_the_same_history(seed):
    """Random forks, growth and frees: inside every group's reported shared
    tokens (and each sequence's length) the group's histories agree."""
    rng = random.Random(100 + seed)
    bm, c = BlockManagerOracle(64, 4), Contents(64, 0, 4)
    hist, tok, next_id = {}, 0, 0
    for _ in range(120):
        live = sorted(bm.tables)
        op = rng.random()
        if op < 0.15 or not live:
            bm.add_sequence(next_id)
            hist[next_id] = []
            next_id += 1
        elif op < 0.35:
            parent = rng.choice(live)
            bm.fork(parent, next_id)
            hist[next_id] = list(hist[parent])
            next_id += 1
        elif op < 0.42 and len(live) > 1:
            s = rng.choice(live)
            bm.free_sequence(s)
            del hist[s]
        else:
            s = rng.choice(live)
            try:
                tok = _grow(bm, c, s, hist, 1, tok)
            except NoFreeBlock:
                pass
        live = sorted(bm.tables)
        for size in (1, 2, 3):
            ids = live[:len(live) // size * size]
            for k, shared in enumerate(bm.shared_prefix(ids, size) if ids else []):
                group = ids[k * size:(k + 1) * size]
                upto = min([shared] + [len(hist[s]) for s in group])
                assert len({tuple(hist[s][:upto]) for s in group}) == 1
                assert shared % 4 == 0
