"""Host block manager: physical block allocation, reference counts, copy-on-write.

The device kernels only consume what this produces: block tables, the slot of
every new token, and the (source, destination) pairs of blocks to copy.

Behaviour follows 0h-n0.github.io, "論文解説: Efficient Memory Management for
Large Language Model Serving with PagedAttention": blocks of ``B`` token
slots, a per-sequence table from logical to physical block numbers (section
"PagedAttentionのメモリ管理"), a reference count per physical block, and the
copy-on-write rule of section "Copy-on-Write（CoW）によるメモリ共有": a write
into a block whose count exceeds one first allocates a new block, copies the
shared block into it, decrements the old block's count and remaps the
sequence's table entry; a block referenced once is written in place.
Forked sequences (parallel samples, beams) share every block of their parent
(dihengye.cn, "PagedAttention", section "KV Cache 共享机制").  Releasing a
sequence drops its references and returns a block to the free list only when
no other sequence still uses it (auturnal.com, "メモリ予算内での言語モデルの
サービング", section 8).
"""

from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    """No free physical block is left."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        """``free_order``: the order in which free blocks are handed out
        (default ascending ids)."""
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the block ids")
        self._free = deque(order)
        self._ref = [0] * self.num_blocks
        self._tables = {}
        self._lens = {}
        self._next_seq = 0

    # ------------------------------------------------------------ blocks
    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted("no free KV block")
        block = self._free.popleft()
        self._ref[block] = 1
        return block

    def ref_count(self, block: int) -> int:
        return self._ref[block]

    def _release(self, block: int):
        if self._ref[block] <= 0:
            raise RuntimeError(f"block {block} released more often than referenced")
        self._ref[block] -= 1
        if self._ref[block] == 0:
            self._free.append(block)

    @property
    def num_free(self) -> int:
        return len(self._free)

    # --------------------------------------------------------- sequences
    def add_sequence(self) -> int:
        seq = self._next_seq
        self._next_seq += 1
        self._tables[seq] = []
        self._lens[seq] = 0
        return seq

    def block_table(self, seq: int):
        return list(self._tables[seq])

    def seq_len(self, seq: int) -> int:
        return self._lens[seq]

    def sequences(self):
        return list(self._tables)

    def fork(self, seq: int, n: int):
        """``n`` new sequences sharing every block (and the length) of ``seq``."""
        children = []
        for _ in range(n):
            child = self.add_sequence()
            self._tables[child] = list(self._tables[seq])
            self._lens[child] = self._lens[seq]
            for b in self._tables[seq]:
                self._ref[b] += 1
            children.append(child)
        return children

    def prepare_write(self, seq: int, logical_block: int):
        """Physical block that ``seq`` may write for ``logical_block``.

        Returns ``(block, pair)``: ``pair`` is ``(src, dst)`` when a copy is
        needed before the write (the block was shared), else ``None``.
        """
        table = self._tables[seq]
        block = table[logical_block]
        if self._ref[block] > 1:
            new_block = self.allocate()
            self._ref[block] -= 1
            table[logical_block] = new_block
            return new_block, (block, new_block)
        return block, None

    def append_slot(self, seq: int):
        """Slot for the sequence's next token, and a copy pair if one is due.

        A new block is taken when the last one is full (or the sequence is
        empty); a shared partially filled last block is copied first.
        """
        pos = self._lens[seq]
        logical = pos // self.block_size
        table = self._tables[seq]
        pair = None
        if logical == len(table):
            table.append(self.allocate())
            block = table[logical]
        else:
            block, pair = self.prepare_write(seq, logical)
        self._lens[seq] = pos + 1
        return block * self.block_size + pos % self.block_size, pair

    def free_sequence(self, seq: int):
        """Drop the sequence and its references (shared blocks stay alive)."""
        for b in self._tables.pop(seq):
            self._release(b)
        del self._lens[seq]

    def tables_array(self, seqs, width=None):
        """int32 ``[len(seqs)][width]`` block tables padded with -1."""
        import numpy as np
        width = width or max(1, max((len(self._tables[s]) for s in seqs), default=1))
        out = np.full((len(seqs), width), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            t = self._tables[s]
            out[i, :len(t)] = t
        return out

    def check_invariants(self):
        """Reference counts equal the number of table entries naming each
        block; no block is both free and referenced."""
        counts = [0] * self.num_blocks
        for t in self._tables.values():
            for b in t:
                counts[b] += 1
        if counts != self._ref:
            raise AssertionError("reference counts disagree with the tables")
        free = set(self._free)
        if len(free) != len(self._free):
            raise AssertionError("a block is on the free list twice")
        for b in free:
            if self._ref[b] != 0:
                raise AssertionError(f"block {b} is free but referenced")
        if len(free) + sum(1 for r in self._ref if r > 0) != self.num_blocks:
            raise AssertionError("a block is neither free nor referenced")
