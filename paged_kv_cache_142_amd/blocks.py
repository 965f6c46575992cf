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

Preemption by swapping (explainer, section "プリエンプション戦略", strategy 1):
``swap_out`` moves a sequence's blocks to a second pool of CPU blocks and
frees its GPU blocks; ``swap_in`` brings them back into free GPU blocks.
Both return the ``(source, destination)`` block pairs that
``pa_swap_blocks`` transfers.  Only sequences that share no block can be
swapped here (a shared block would have to stay where its other users read
it).
"""

from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    """No free physical block is left."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None, num_cpu_blocks: int = 0):
        """``free_order``: the order in which free blocks are handed out
        (default ascending ids).  ``num_cpu_blocks``: size of the CPU pool
        that swapped-out sequences occupy."""
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
        self.num_cpu_blocks = int(num_cpu_blocks)
        self._cpu_free = deque(range(self.num_cpu_blocks))
        self._swapped = {}  # seq -> CPU block table

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
        """Drop the sequence and its references (shared blocks stay alive);
        a swapped-out sequence returns its CPU blocks."""
        if seq in self._swapped:
            self._cpu_free.extend(self._swapped.pop(seq))
        else:
            for b in self._tables.pop(seq):
                self._release(b)
        del self._lens[seq]

    # ---------------------------------------------------------- swapping
    def swap_out(self, seq: int):
        """Move the sequence to CPU blocks.  Returns the ``(gpu, cpu)`` pairs
        to transfer (device pool -> host pool); its GPU blocks are free
        afterwards and the sequence has no table until ``swap_in``."""
        table = self._tables[seq]
        if any(self._ref[b] != 1 for b in table):
            raise RuntimeError(f"sequence {seq} shares blocks and cannot be swapped out alone")
        if len(self._cpu_free) < len(table):
            raise PoolExhausted("no free CPU block")
        cpu = [self._cpu_free.popleft() for _ in table]
        pairs = list(zip(table, cpu))
        for b in table:
            self._release(b)
        del self._tables[seq]
        self._swapped[seq] = cpu
        return pairs

    def swap_in(self, seq: int):
        """Bring a swapped-out sequence back into free GPU blocks.  Returns the
        ``(cpu, gpu)`` pairs to transfer (host pool -> device pool)."""
        cpu = self._swapped[seq]
        if len(self._free) < len(cpu):
            raise PoolExhausted("no free KV block")
        gpu = [self.allocate() for _ in cpu]
        del self._swapped[seq]
        self._cpu_free.extend(cpu)
        self._tables[seq] = gpu
        return list(zip(cpu, gpu))

    def is_swapped(self, seq: int) -> bool:
        return seq in self._swapped

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
        held = [b for t in self._swapped.values() for b in t]
        if len(set(held)) != len(held) or set(held) & set(self._cpu_free) or \
                len(held) + len(self._cpu_free) != self.num_cpu_blocks:
            raise AssertionError("CPU blocks are not partitioned into held and free")
