"""ctypes binding of the host block manager (include/pkv_block_manager.h).

Argument marshalling only; the bookkeeping runs in libpkv.so (C++).
"""

from __future__ import annotations

import ctypes

import numpy as np

from ._lib import PkvError, library, status_string

_BOUND = False


def _bind():
    global _BOUND
    if _BOUND:
        return library()
    lib = library()
    P, I, L = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.pkv_bm_create.argtypes = [I, I]
    lib.pkv_bm_create.restype = P
    lib.pkv_bm_create_swappable.argtypes = [I, I, I]
    lib.pkv_bm_create_swappable.restype = P
    lib.pkv_bm_destroy.argtypes = [P]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_add_sequence.argtypes = [P, L]
    lib.pkv_bm_fork.argtypes = [P, L, L]
    lib.pkv_bm_append_token.argtypes = [P, L, P, P]
    lib.pkv_bm_append_batch.argtypes = [P, P, I, P, P]
    lib.pkv_bm_free_sequence.argtypes = [P, L]
    lib.pkv_bm_num_free_blocks.argtypes = [P]
    lib.pkv_bm_seq_len.argtypes = [P, L]
    lib.pkv_bm_refcount.argtypes = [P, ctypes.c_int32]
    lib.pkv_bm_block_table.argtypes = [P, L, P, I]
    lib.pkv_bm_take_copies.argtypes = [P, P, I]
    lib.pkv_bm_build_batch.argtypes = [P, P, I, P, I, P]
    lib.pkv_bm_shared_prefix.argtypes = [P, P, I, I, P]
    lib.pkv_bm_swap_out.argtypes = [P, P, I, P, I]
    lib.pkv_bm_swap_in.argtypes = [P, P, I, P, I]
    lib.pkv_bm_is_swapped.argtypes = [P, L]
    lib.pkv_bm_num_free_host_blocks.argtypes = [P]
    lib.pkv_bm_host_refcount.argtypes = [P, ctypes.c_int32]
    for name in ("pkv_bm_add_sequence", "pkv_bm_fork", "pkv_bm_append_token", "pkv_bm_append_batch",
                 "pkv_bm_free_sequence", "pkv_bm_num_free_blocks", "pkv_bm_seq_len",
                 "pkv_bm_refcount", "pkv_bm_block_table", "pkv_bm_take_copies",
                 "pkv_bm_build_batch", "pkv_bm_swap_out", "pkv_bm_swap_in", "pkv_bm_is_swapped",
                 "pkv_bm_num_free_host_blocks", "pkv_bm_host_refcount", "pkv_bm_shared_prefix"):
        getattr(lib, name).restype = I
    _BOUND = True
    return lib


def _check(fn, status):
    if status < 0:
        raise PkvError(fn, status, status_string(status))
    return status


class BlockManager:
    """Blocks of a pool of num_blocks blocks of block_size tokens: on-demand
    allocation, shared blocks with reference counts, copy-on-write, and
    swapping of sequences to a pool of num_host_blocks host blocks."""

    def __init__(self, num_blocks: int, block_size: int, num_host_blocks: int = 0):
        self._lib = _bind()
        self._h = self._lib.pkv_bm_create_swappable(int(num_blocks), int(num_host_blocks),
                                                    int(block_size))
        if not self._h:
            raise ValueError("invalid pool size or block size")
        self.num_blocks = int(num_blocks)
        self.num_host_blocks = int(num_host_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pkv_bm_destroy(h)

    def add_sequence(self, seq_id: int) -> None:
        _check("pkv_bm_add_sequence", self._lib.pkv_bm_add_sequence(self._h, seq_id))

    def fork(self, parent: int, child: int) -> None:
        _check("pkv_bm_fork", self._lib.pkv_bm_fork(self._h, parent, child))

    def append_token(self, seq_id: int) -> tuple[int, int]:
        """Reserve the next token's slot; returns (physical block, offset)."""
        b, o = ctypes.c_int32(), ctypes.c_int32()
        _check("pkv_bm_append_token", self._lib.pkv_bm_append_token(
            self._h, seq_id, ctypes.byref(b), ctypes.byref(o)))
        return b.value, o.value

    def append_batch(self, seq_ids) -> tuple[np.ndarray, np.ndarray]:
        """append_token for every id in order, all or nothing; returns the
        (blocks, offsets) arrays."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        blocks = np.empty(len(ids), dtype=np.int32)
        offsets = np.empty(len(ids), dtype=np.int32)
        _check("pkv_bm_append_batch", self._lib.pkv_bm_append_batch(
            self._h, ids.ctypes.data, len(ids), blocks.ctypes.data, offsets.ctypes.data))
        return blocks, offsets

    def free_sequence(self, seq_id: int) -> None:
        _check("pkv_bm_free_sequence", self._lib.pkv_bm_free_sequence(self._h, seq_id))

    def num_free_blocks(self) -> int:
        return _check("pkv_bm_num_free_blocks", self._lib.pkv_bm_num_free_blocks(self._h))

    def seq_len(self, seq_id: int) -> int:
        return _check("pkv_bm_seq_len", self._lib.pkv_bm_seq_len(self._h, seq_id))

    def refcount(self, block: int) -> int:
        return _check("pkv_bm_refcount", self._lib.pkv_bm_refcount(self._h, block))

    def block_table(self, seq_id: int) -> list[int]:
        """Logical -> physical blocks (host blocks if the sequence is swapped out)."""
        cap = max(self.num_blocks, self.num_host_blocks)
        buf = np.empty(cap, dtype=np.int32)
        n = _check("pkv_bm_block_table", self._lib.pkv_bm_block_table(
            self._h, seq_id, buf.ctypes.data, cap))
        return buf[:n].tolist()

    def _move(self, fn: str, seq_ids, capacity: int) -> np.ndarray:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        pairs = np.empty((max(capacity, 1), 2), dtype=np.int32)
        n = _check(fn, getattr(self._lib, fn)(self._h, ids.ctypes.data, len(ids),
                                              pairs.ctypes.data, capacity))
        return pairs[:n].copy()

    def swap_out(self, seq_ids) -> np.ndarray:
        """Move the sequences to host blocks, all or nothing; returns the
        int32 [P][2] (device block, host block) pairs to copy."""
        return self._move("pkv_bm_swap_out", seq_ids, self.num_blocks)

    def swap_in(self, seq_ids) -> np.ndarray:
        """Bring swapped-out sequences back, all or nothing; returns the
        int32 [P][2] (host block, device block) pairs to copy."""
        return self._move("pkv_bm_swap_in", seq_ids, self.num_host_blocks)

    def is_swapped(self, seq_id: int) -> bool:
        return bool(_check("pkv_bm_is_swapped", self._lib.pkv_bm_is_swapped(self._h, seq_id)))

    def num_free_host_blocks(self) -> int:
        return _check("pkv_bm_num_free_host_blocks",
                      self._lib.pkv_bm_num_free_host_blocks(self._h))

    def host_refcount(self, block: int) -> int:
        return _check("pkv_bm_host_refcount", self._lib.pkv_bm_host_refcount(self._h, block))

    def take_copies(self) -> np.ndarray:
        """Queued copy-on-write pairs, int32 [P][2] (src, dst), in order."""
        buf = np.empty((self.num_blocks, 2), dtype=np.int32)
        out = []
        while True:
            n = _check("pkv_bm_take_copies", self._lib.pkv_bm_take_copies(
                self._h, buf.ctypes.data, buf.shape[0]))
            out.append(buf[:n].copy())
            if n < buf.shape[0]:
                break
        return np.concatenate(out).reshape(-1, 2)

    def shared_prefix(self, seq_ids, group_size: int) -> np.ndarray:
        """int32 [n // group_size]: per group of group_size consecutive ids, the
        tokens of the leading blocks all its sequences share."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        out = np.empty(max(len(ids) // max(group_size, 1), 1), dtype=np.int32)
        _check("pkv_bm_shared_prefix", self._lib.pkv_bm_shared_prefix(
            self._h, ids.ctypes.data, len(ids), int(group_size), out.ctypes.data))
        return out[:len(ids) // group_size]

    def build_batch(self, seq_ids, max_blocks: int) -> tuple[np.ndarray, np.ndarray]:
        """int32 block tables [n][max_blocks] (padded with -1) and seq_lens [n]."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        tables = np.empty((len(ids), max_blocks), dtype=np.int32)
        lens = np.empty(len(ids), dtype=np.int32)
        _check("pkv_bm_build_batch", self._lib.pkv_bm_build_batch(
            self._h, ids.ctypes.data, len(ids), tables.ctypes.data, int(max_blocks),
            lens.ctypes.data))
        return tables, lens
