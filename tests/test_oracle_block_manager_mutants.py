"""Plausible mistakes planted in the oracle block manager; each must make at
least one pin of tests/test_oracle_block_manager.py fail."""

import pytest

import oracle.block_manager as obm
from tests import test_oracle_block_manager as pins

PINS = [name for name in dir(pins) if name.startswith("test_")]


class CopyEvenWhenFull(obm.BlockManagerOracle):
    def append_token(self, seq):
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


MUTANTS = {c.__name__: c for c in
           (CopyEvenWhenFull, NoDecrementOnCopy, CopyOnEveryPartialWrite, BlockPerToken,
            FreeInReverse)}


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
            except Exception:
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_block_manager_pins_catch_mutant(mutant, monkeypatch):
    monkeypatch.setattr(pins, "BlockManagerOracle", MUTANTS[mutant])
    assert _failing(), f"no pin catches {mutant}"


def test_unmutated_block_manager_passes_every_pin():
    assert _failing() == []
