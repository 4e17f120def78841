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

Swapping (supersilo.blog summary, section "적용 범위와 관련 연구": when
memory runs short, sequences move to CPU memory and come back later). The
pages give no mechanism; the reading taken here:
* a second pool of host blocks with its own free stack (same policy) and
  reference counts;
* swapping out a set of sequences gives every distinct device block they
  hold one host block (a block shared inside the set moves once and stays
  shared), in order of first use (the sequences in the given order, each
  table in logical order); their device references are then dropped as if
  the sequences were freed, in the same order. Swapping in is the mirror
  image. Both are all or nothing;
* a swapped-out sequence cannot grow or be forked until it is swapped in; it
  can be freed;
* copy-on-write copies still queued would be overtaken by the swap's own
  copies, so a swap is refused until they have been taken.

Freeing a sequence is refused while copy-on-write copies are queued (the
pages say nothing on it): a block it releases could be handed out again
before the copies run, as the destination of a second copy of the same step
(two copies writing one block) or as a destination while it is still a
queued copy's source (the copies of one step run concurrently).
"""


class NoFreeBlock(Exception):
    pass


class BlockManagerOracle:
    def __init__(self, num_blocks, block_size, num_host_blocks=0):
        self.block_size = block_size
        self.free = list(range(num_blocks - 1, -1, -1))     # top of the stack = end
        self.ref = [0] * num_blocks
        self.host_free = list(range(num_host_blocks - 1, -1, -1))
        self.host_ref = [0] * num_host_blocks
        self.tables = {}                                     # seq id -> [physical blocks]
        self.lens = {}
        self.copies = []
        self.swapped = set()                                 # ids whose table names host blocks

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
        assert parent not in self.swapped
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def append_token(self, seq):
        """Reserve the slot of the sequence's next token; returns (block, offset)."""
        assert seq not in self.swapped
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
        # refused while copy-on-write copies are queued: a freed block could
        # be handed out again, before the copies run, as the destination of
        # a second copy or as a destination while still a copy's source
        assert not self.copies, "queued copy-on-write copies must be taken first"
        ref, free = (self.host_ref, self.host_free) if seq in self.swapped else (self.ref, self.free)
        for b in self.tables.pop(seq):
            ref[b] -= 1
            if ref[b] == 0:
                free.append(b)
        del self.lens[seq]
        self.swapped.discard(seq)

    def _move(self, seqs, to_host):
        """Give every distinct block of `seqs` a block of the other pool;
        returns the (old block, new block) pairs in order of first use."""
        seqs = list(seqs)
        assert len(set(seqs)) == len(seqs)
        assert all(s in self.tables and (s in self.swapped) != to_host for s in seqs)
        assert not self.copies, "queued copy-on-write copies must be taken first"
        src_ref, src_free = (self.ref, self.free) if to_host else (self.host_ref, self.host_free)
        dst_ref, dst_free = (self.host_ref, self.host_free) if to_host else (self.ref, self.free)
        order = []
        for s in seqs:
            for b in self.tables[s]:
                if b not in order:
                    order.append(b)
        if len(order) > len(dst_free):
            raise NoFreeBlock()
        where = {}
        for b in order:
            where[b] = dst_free.pop()
            dst_ref[where[b]] = 0
        for s in seqs:
            for b in self.tables[s]:
                dst_ref[where[b]] += 1
                src_ref[b] -= 1
                if src_ref[b] == 0:
                    src_free.append(b)
            self.tables[s] = [where[b] for b in self.tables[s]]
            if to_host:
                self.swapped.add(s)
            else:
                self.swapped.discard(s)
        return [(b, where[b]) for b in order]

    def shared_prefix(self, seqs, group_size):
        """Per group of group_size consecutive ids: block_size times the number
        of leading logical blocks every sequence of the group maps to the same
        physical block."""
        seqs = list(seqs)
        assert len(seqs) % group_size == 0
        assert all(s in self.tables and s not in self.swapped for s in seqs)
        out = []
        for k in range(0, len(seqs), group_size):
            tables = [self.tables[s] for s in seqs[k:k + group_size]]
            b = 0
            while all(b < len(t) for t in tables) and len({t[b] for t in tables}) == 1:
                b += 1
            out.append(b * self.block_size)
        return out

    def swap_out(self, seqs):
        """Move resident sequences to host blocks; returns the (device block,
        host block) pairs whose contents must be copied device -> host."""
        return self._move(seqs, to_host=True)

    def swap_in(self, seqs):
        """Bring swapped-out sequences back; returns the (host block, device
        block) pairs whose contents must be copied host -> device."""
        return self._move(seqs, to_host=False)

    def take_copies(self):
        out, self.copies = self.copies, []
        return out
