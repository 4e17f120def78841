"""Plausible mistakes planted in the oracle block manager; each must make at
least one pin of tests/test_oracle_block_manager.py fail."""

import pytest

import oracle.block_manager as obm
from tests import test_oracle_block_manager as pins

PINS = [name for name in dir(pins) if name.startswith("test_")]


class CopyEvenWhenFull(obm.BlockManagerOracle):
    def append_token(self, seq):
        assert seq not in self.swapped
        table = self.tables[seq]
        offset = self.lens[seq] % self.block_size
        if table and self.ref[table[-1]] > 1:
            old = table[-1]
            new = self._take()
            self.copies.append((old, new))
            self.ref[old] -= 1
            table[-1] = new
        if offset == 0:
            table.append(self._take())
        self.lens[seq] += 1
        return table[-1], offset


class NoDecrementOnCopy(obm.BlockManagerOracle):
    def append_token(self, seq):
        assert seq not in self.swapped
        table = self.tables[seq]
        offset = self.lens[seq] % self.block_size
        if offset == 0:
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            old = table[-1]
            new = self._take()
            self.copies.append((old, new))
            table[-1] = new
        self.lens[seq] += 1
        return table[-1], offset


class CopyOnEveryPartialWrite(obm.BlockManagerOracle):
    """Copies a partly filled last block on every write, shared or not."""
    def append_token(self, seq):
        assert seq not in self.swapped
        table = self.tables[seq]
        offset = self.lens[seq] % self.block_size
        if offset == 0:
            table.append(self._take())
        else:
            old = table[-1]
            new = self._take()
            self.copies.append((old, new))
            self.ref[old] -= 1
            if self.ref[old] == 0:
                self.free.append(old)
            table[-1] = new
        self.lens[seq] += 1
        return table[-1], offset


class BlockPerToken(obm.BlockManagerOracle):
    def append_token(self, seq):
        assert seq not in self.swapped
        self.tables[seq].append(self._take())
        self.lens[seq] += 1
        return self.tables[seq][-1], 0


class FreeInReverse(obm.BlockManagerOracle):
    def free_sequence(self, seq):
        for b in reversed(self.tables.pop(seq)):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]


class SwapKeepsDeviceBlocks(obm.BlockManagerOracle):
    """Swapping out does not give the device blocks back."""
    def swap_out(self, seqs):
        ref, free = list(self.ref), list(self.free)
        pairs = super().swap_out(seqs)
        self.ref, self.free = ref, free
        return pairs


class SwapEveryReference(obm.BlockManagerOracle):
    """One host block per table entry: a shared block moves once per holder."""
    def _move(self, seqs, to_host):
        pairs = []
        for s in seqs:
            pairs += super()._move([s], to_host)
        return pairs


class SwapInPairsBackwards(obm.BlockManagerOracle):
    """Swap-in pairs name (device, host) instead of (host, device)."""
    def swap_in(self, seqs):
        return [(d, h) for h, d in super().swap_in(seqs)]


class SwapPartly(obm.BlockManagerOracle):
    """Moves the leading sequences that fit instead of refusing the set."""
    def _move(self, seqs, to_host):
        seqs = list(seqs)
        while seqs:
            try:
                return super()._move(seqs, to_host)
            except obm.NoFreeBlock:
                seqs.pop()
        return []


class SwapForgetsTheHostSide(obm.BlockManagerOracle):
    """Swapping in never gives the host blocks back."""
    def swap_in(self, seqs):
        host_ref, host_free = list(self.host_ref), list(self.host_free)
        pairs = super().swap_in(seqs)
        self.host_ref, self.host_free = host_ref, host_free
        return pairs


class SharedByTheFirstTwo(obm.BlockManagerOracle):
    """Compares only the first two sequences of a group."""
    def shared_prefix(self, seqs, group_size):
        seqs = list(seqs)
        out = []
        for k in range(0, len(seqs), group_size):
            pair = seqs[k:k + min(2, group_size)]
            out += super().shared_prefix(pair, len(pair))
        return out


class SharedCountsAllBlocks(obm.BlockManagerOracle):
    """Counts every block any sequence of the group shares with the first."""
    def shared_prefix(self, seqs, group_size):
        seqs = list(seqs)
        out = []
        for k in range(0, len(seqs), group_size):
            first = self.tables[seqs[k]]
            n = max(sum(1 for b in range(min(len(first), len(self.tables[s])))
                        if self.tables[s][b] == first[b]) for s in seqs[k:k + group_size])
            out.append(n * self.block_size)
        return out


MUTANTS = {c.__name__: c for c in
           (CopyEvenWhenFull, NoDecrementOnCopy, CopyOnEveryPartialWrite, BlockPerToken,
            FreeInReverse, SwapKeepsDeviceBlocks, SwapEveryReference, SwapInPairsBackwards,
            SwapPartly, SwapForgetsTheHostSide, SharedByTheFirstTwo, SharedCountsAllBlocks)}


def _failing():
    failed = []
    for name in PINS:
        fn = getattr(pins, name)
        args = [()]
        for m in getattr(fn, "pytestmark", []):
            if m.name == "parametrize":
                args = [(v,) for v in m.args[1]]
        for a in args:
            try:
                fn(*a)
            except (Exception, pytest.fail.Exception):
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_block_manager_pins_catch_mutant(mutant, monkeypatch):
    monkeypatch.setattr(pins, "BlockManagerOracle", MUTANTS[mutant])
    assert _failing(), f"no pin catches {mutant}"


def test_unmutated_block_manager_passes_every_pin():
    assert _failing() == []
