"""Plain Python block manager: what the host does before each decode step.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

From the pages (supersilo.blog vLLM/PagedAttention summary, sections
"PagedAttention의 설계" and "블록 공유"; blog.aqudi.me "벤치마크가 다가
아니야! vLLM으로 보는 LLM 추론 최적화", section 3; hjr-study-book Day 3,
section 4.2):
* the block manager hands out fixed-size blocks and takes them back; a
  request gets a new block only when its current one is full, so the waste
  of a sequence is confined to its last block;
* sequences that start from the same prompt (parallel sampling, beam search)
  point at the same physical blocks;
* a shared block is copied only at the moment one holder must modify it
  (copy-on-write).

Readings where the pages are silent:
* "must modify" = appending a token into a shared block that still has free
  slots; a full shared block is never written again, so the writer gets a
  fresh block and no copy. The last remaining holder writes in place.
* Allocation order (any free block would do; a fixed rule makes results
  comparable): free blocks form a stack with block 0 on top, then 1, 2, ...;
  freed blocks are pushed on top, a sequence's blocks in logical order.
"""


class NoFreeBlock(Exception):
    pass


class BlockManagerOracle:
    def __init__(self, num_blocks, block_size):
        self.block_size = block_size
        self.free = list(range(num_blocks - 1, -1, -1))     # top of the stack = end
        self.ref = [0] * num_blocks
        self.tables = {}                                     # seq id -> [physical blocks]
        self.lens = {}
        self.copies = []

    def _take(self):
        if not self.free:
            raise NoFreeBlock()
        b = self.free.pop()
        self.ref[b] = 1
        return b

    def add_sequence(self, seq):
        assert seq not in self.tables
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent, child):
        assert child not in self.tables and parent in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_token(self, seq):
        """Reserve the slot of the sequence's next token; returns (block, offset)."""
        table = self.tables[seq]
        offset = self.lens[seq] % self.block_size
        if offset == 0:
            table.append(self._take())
        elif self.ref[table[-1]] > 1:
            old = table[-1]
            new = self._take()
            self.copies.append((old, new))
            self.ref[old] -= 1
            table[-1] = new
        self.lens[seq] += 1
        return table[-1], offset

    def free_sequence(self, seq):
        for b in self.tables.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def take_copies(self):
        out, self.copies = self.copies, []
        return out
