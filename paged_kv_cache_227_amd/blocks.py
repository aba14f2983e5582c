"""Host-side block manager: the free list, reference counts and per-sequence
block tables that the GPU path consumes.

Semantics follow the two allocators on the pages:

* "How a serving engine actually works" (paperfordummies.in), section
  "The code": a FIFO free list (allocate takes the front, a freed block goes to
  the back), a refcount per block, ``share`` as a refcount bump, the guard that
  only the last owner really frees, copy-on-write, and ``OutOfBlocks`` when the
  pool is empty.  The ``Sequence`` class there (a table plus a length that grows
  a block when the current one is full, ``fork``, ``release``) is mirrored here.
* "Paged Attention and the Block Manager" (snowch.github.io ch08), section
  "The build": ``ValueError`` for a non-positive pool or block size,
  ``blocks_needed`` and ``allocate(n)`` returning a list, ``n_free``.
* "Paged-KV + Continuous Batching From Scratch" (henryhe.ai), section 2: the
  allocator hard-fails on a double free.

Unlike the pages' counter simulation, ``copy_on_write`` here reports the block
whose rows the caller must copy (the simulation allocates without copying any
data); copying the rows is the caller's job.  ``Sequence`` queues each such copy
as (source block, private block, rows already written); ``take_copies`` hands
the queue to the caller, who runs them (``paged_kv_copy_blocks``) before the
append that triggered them.

This module does bookkeeping only; it never touches device memory.
"""
from __future__ import annotations

from typing import Iterable, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    """No free physical block is left in the pool."""


class DoubleFree(RuntimeError):
    """A block was released more times than it was referenced."""


class BlockAllocator:
    """A pool of ``n_blocks`` fixed-size KV blocks with reference counts."""

    def __init__(self, n_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None) -> None:
        if n_blocks < 1 or block_size < 1:
            raise ValueError("n_blocks and block_size must both be positive")
        self.n_blocks = int(n_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            self._free: List[int] = list(range(self.n_blocks))
        else:
            self._free = [int(b) for b in free_order]
            if sorted(self._free) != list(range(self.n_blocks)):
                raise ValueError("free_order must be a permutation of range(n_blocks)")
        self._ref: dict = {}
        self.copies = 0  # copy-on-write events

    # -- queries ---------------------------------------------------------
    @property
    def n_free(self) -> int:
        return len(self._free)

    @property
    def free_list(self) -> List[int]:
        return list(self._free)

    def refcount(self, b: int) -> int:
        return self._ref.get(b, 0)

    def blocks_needed(self, n_tokens: int) -> int:
        """Blocks that hold ``n_tokens`` tokens: the ceiling of n_tokens / block_size."""
        return -(-int(n_tokens) // self.block_size)

    # -- allocation ------------------------------------------------------
    def allocate_one(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free physical blocks")
        b = self._free.pop(0)
        self._ref[b] = 1
        return b

    def allocate(self, n: int) -> List[int]:
        """``n`` blocks, all or none."""
        if n < 0:
            raise ValueError("cannot allocate a negative number of blocks")
        if n > len(self._free):
            raise OutOfBlocks("no free physical blocks")
        return [self.allocate_one() for _ in range(n)]

    def share(self, b: int) -> int:
        """Another sequence now points at block ``b``; nothing is copied."""
        if b not in self._ref:
            raise DoubleFree("share of block %d, which is not allocated" % b)
        self._ref[b] += 1
        return b

    def free_block(self, b: int) -> bool:
        """Drop one reference; return True when the block went back to the pool."""
        if b not in self._ref:
            raise DoubleFree("block %d released more often than referenced" % b)
        self._ref[b] -= 1
        if self._ref[b] == 0:
            del self._ref[b]
            self._free.append(b)
            return True
        return False

    def copy_on_write(self, b: int) -> int:
        """Block to write into instead of ``b``: ``b`` itself if this is its sole
        owner, otherwise a fresh private block (the caller copies ``b``'s rows)."""
        if b not in self._ref:
            raise DoubleFree("write into block %d, which is not allocated" % b)
        if self._ref[b] == 1:
            return b
        new = self.allocate_one()
        self._ref[b] -= 1
        self.copies += 1
        return new

    def is_whole(self) -> bool:
        """True when every block is free again (no leak)."""
        return not self._ref and sorted(self._free) == list(range(self.n_blocks))


class Sequence:
    """A block table plus a length."""

    def __init__(self, name: str, alloc: BlockAllocator) -> None:
        self.name = name
        self.alloc = alloc
        self.table: List[int] = []
        self.n_tokens = 0
        self.last_cow: Optional[tuple] = None  # (src, dst) of the latest private copy
        self.pending_copies: List[Tuple[int, int, int]] = []  # (src, dst, rows) not yet run

    def append_tokens(self, n: int) -> None:
        """Grow by ``n`` tokens: a new block when the current one is full, a
        private copy when writing inside a block someone else also holds."""
        for _ in range(n):
            offset = self.n_tokens % self.alloc.block_size
            if offset == 0:
                self.table.append(self.alloc.allocate_one())
            else:
                last = len(self.table) - 1
                old = self.table[last]
                new = self.alloc.copy_on_write(old)
                if new != old:
                    self.last_cow = (old, new)
                    # rows 0 .. offset-1 hold this sequence's tokens already
                    self.pending_copies.append((old, new, offset))
                self.table[last] = new
            self.n_tokens += 1

    def take_copies(self) -> List[Tuple[int, int, int]]:
        """The queued (src, dst, rows) block copies, oldest first; clears the queue."""
        out, self.pending_copies = self.pending_copies, []
        return out

    def fork(self, name: str) -> "Sequence":
        """Same tokens, shared blocks (parallel sampling, shared prompts)."""
        child = Sequence(name, self.alloc)
        child.table = [self.alloc.share(b) for b in self.table]
        child.n_tokens = self.n_tokens
        return child

    def preempt_swap(self) -> List[int]:
        """Preemption by swapping, all or nothing: the blocks whose contents the
        caller copies to host memory (table order), after which every one is
        released.  The tokens stay (``n_tokens`` is kept); only the cache leaves."""
        blocks = list(self.table)
        for b in blocks:
            self.alloc.free_block(b)
        self.table = []
        return blocks

    def resume_swapped(self, n_blocks: int) -> List[int]:
        """Fresh blocks for a swapped-out sequence, all or none; host slot i goes
        into the i-th returned block.  Blocks it once shared come back private."""
        if n_blocks != self.alloc.blocks_needed(self.n_tokens):
            raise ValueError("a swapped-out sequence of %d tokens needs %d blocks, not %d"
                             % (self.n_tokens, self.alloc.blocks_needed(self.n_tokens), n_blocks))
        self.table = self.alloc.allocate(n_blocks)
        return list(self.table)

    def release(self) -> None:
        for b in self.table:
            self.alloc.free_block(b)
        self.table = []
        self.n_tokens = 0

    def internal_waste(self) -> int:
        """Slots held but not written: at most block_size - 1."""
        return len(self.table) * self.alloc.block_size - self.n_tokens
