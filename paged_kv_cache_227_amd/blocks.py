"""Host-side bookkeeping for the paged cache: which physical blocks are idle,
how many block tables point at each block, and each sequence's table.  The GPU
path only ever sees the resulting tables; this module never touches device
memory.

The rules it keeps are the ones the pages state:

* "How a serving engine actually works" (paperfordummies.in), "The code":
  blocks are reused first-freed-first-reused; sharing a block only counts one
  more holder; a block goes back to the pool when its last holder lets go;
  writing into a block that others also hold first moves the writer to a
  private block; an empty pool is an error (``OutOfBlocks``).
* "Paged Attention and the Block Manager" (snowch.github.io ch08), "The build":
  a pool of no blocks, or of empty blocks, is a ``ValueError``; a request for
  n blocks is served whole or not at all.
* "Paged-KV + Continuous Batching From Scratch" (henryhe.ai), section 2: giving
  back a block that nobody holds is a hard failure (``DoubleFree``).

Design.  The pool is two structures: ``_holders``, one count per physical
block (zero means idle), and ``_idle``, a deque of the idle block ids in the
order they became idle.  Every operation is a few O(1) steps on them.  A
sequence is a list of block ids plus its token count; the slot of its token i
is ``table[i // B] * B + i % B``.

Where the pages' simulation only counts a copy-on-write, here the writer's
``Sequence`` also queues the data move it implies (source block, private
block, rows already written) for the caller to run on the device
(``paged_kv_copy_blocks``) before the append that caused it.
"""
from __future__ import annotations

from collections import deque
from typing import Iterable, List, Optional, Tuple


class OutOfBlocks(RuntimeError):
    """The pool has fewer idle blocks than a request needs."""


class DoubleFree(RuntimeError):
    """An operation named a block that no table holds."""


class BlockAllocator:
    """``n_blocks`` physical blocks of ``block_size`` token slots each.

    ``free_order`` fixes the order in which the idle blocks are first handed
    out (a permutation of the block ids); by default it is 0, 1, 2, ...
    ``copies`` counts the private blocks handed out by ``copy_on_write``.
    """

    def __init__(self, n_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None) -> None:
        n_blocks, block_size = int(n_blocks), int(block_size)
        if n_blocks <= 0 or block_size <= 0:
            raise ValueError("a pool needs at least one block of at least one slot "
                             "(got %d blocks of %d)" % (n_blocks, block_size))
        ids = list(range(n_blocks)) if free_order is None else [int(b) for b in free_order]
        if len(ids) != n_blocks or set(ids) != set(range(n_blocks)):
            raise ValueError("free_order must list every block id 0..%d exactly once" % (n_blocks - 1))
        self.n_blocks = n_blocks
        self.block_size = block_size
        self._holders = [0] * n_blocks
        self._idle = deque(ids)
        self.copies = 0

    # ---- state ------------------------------------------------------------
    @property
    def n_free(self) -> int:
        return len(self._idle)

    @property
    def free_list(self) -> List[int]:
        """Idle block ids, next to be handed out first."""
        return list(self._idle)

    def refcount(self, b: int) -> int:
        return self._holders[b] if 0 <= b < self.n_blocks else 0

    def blocks_needed(self, n_tokens: int) -> int:
        """Blocks a table needs for ``n_tokens`` tokens (n_tokens / B rounded up)."""
        n_tokens = int(n_tokens)
        return (n_tokens + self.block_size - 1) // self.block_size

    def is_whole(self) -> bool:
        """Every block idle and listed once: nothing leaked, nothing listed twice."""
        return not any(self._holders) and sorted(self._idle) == list(range(self.n_blocks))

    def _check_held(self, b: int, op: str) -> None:
        if not (0 <= b < self.n_blocks) or self._holders[b] == 0:
            raise DoubleFree("%s: block %d has no holder" % (op, b))

    # ---- operations -------------------------------------------------------
    def allocate(self, n: int) -> List[int]:
        """Hand out the ``n`` longest-idle blocks, each with one holder; if fewer
        than ``n`` are idle, raise ``OutOfBlocks`` and change nothing."""
        n = int(n)
        if n < 0:
            raise ValueError("block count %d is negative" % n)
        if n > len(self._idle):
            raise OutOfBlocks("pool exhausted: %d block(s) wanted, %d idle" % (n, len(self._idle)))
        out = []
        for _ in range(n):
            b = self._idle.popleft()
            self._holders[b] = 1
            out.append(b)
        return out

    def allocate_one(self) -> int:
        return self.allocate(1)[0]

    def share(self, b: int) -> int:
        """Count one more holder of ``b`` (a forked table pointing at it)."""
        self._check_held(b, "share")
        self._holders[b] += 1
        return b

    def free_block(self, b: int) -> bool:
        """One holder lets go of ``b``; True if that made it idle again."""
        self._check_held(b, "release")
        left = self._holders[b] - 1
        self._holders[b] = left
        if left:
            return False
        self._idle.append(b)
        return True

    def copy_on_write(self, b: int) -> int:
        """The block a holder of ``b`` may write into: ``b`` when it is the only
        holder, else a new private block, the writer giving up its hold on ``b``.
        Moving the rows already written into the private block is the caller's
        job."""
        self._check_held(b, "write")
        if self._holders[b] == 1:
            return b
        private = self.allocate_one()  # may raise before b's count changes
        self.free_block(b)             # others still hold b: it stays live
        self.copies += 1
        return private


class Sequence:
    """One request's block table and the number of tokens it has written.

    ``pending_copies`` queues (source, private, rows) moves that copy-on-write
    made necessary; ``last_cow`` is the latest (source, private) pair.
    """

    def __init__(self, name: str, alloc: BlockAllocator) -> None:
        self.name = name
        self.alloc = alloc
        self.table: List[int] = []
        self.n_tokens = 0
        self.last_cow: Optional[Tuple[int, int]] = None
        self.pending_copies: List[Tuple[int, int, int]] = []

    def _own_next_slot(self) -> None:
        """Make the slot of token ``n_tokens`` exist and be this table's alone."""
        written = self.n_tokens % self.alloc.block_size
        if written == 0:
            # every block in the table is full (or there is none): open one
            self.table.append(self.alloc.allocate_one())
            return
        shared = self.table[-1]
        private = self.alloc.copy_on_write(shared)
        if private != shared:
            self.table[-1] = private
            self.last_cow = (shared, private)
            self.pending_copies.append((shared, private, written))

    def append_tokens(self, n: int) -> None:
        """Reserve slots for ``n`` more tokens, one at a time, so an
        ``OutOfBlocks`` leaves the tokens reserved so far in place."""
        for _ in range(int(n)):
            self._own_next_slot()
            self.n_tokens += 1

    def take_copies(self) -> List[Tuple[int, int, int]]:
        """Hand over the queued block moves, oldest first, and empty the queue."""
        queued = self.pending_copies
        self.pending_copies = []
        return queued

    def fork(self, name: str) -> "Sequence":
        """A new sequence with the same tokens, holding the same blocks."""
        twin = Sequence(name, self.alloc)
        for b in self.table:
            self.alloc.share(b)
        twin.table = list(self.table)
        twin.n_tokens = self.n_tokens
        return twin

    def _let_go(self) -> List[int]:
        dropped = self.table
        self.table = []
        for b in dropped:
            self.alloc.free_block(b)
        return dropped

    def release(self) -> None:
        """Finished: give every block back and forget the tokens."""
        self._let_go()
        self.n_tokens = 0

    def preempt_swap(self) -> List[int]:
        """Preemption by swapping: returns the table (in order) whose blocks the
        caller copies to host memory, then gives every block back.  The token
        count stays, so the sequence can resume where it stopped."""
        return list(self._let_go())

    def resume_swapped(self, n_blocks: int) -> List[int]:
        """New private blocks for a swapped-out sequence, all or none; host
        slot i is copied into the i-th one returned."""
        want = self.alloc.blocks_needed(self.n_tokens)
        if int(n_blocks) != want:
            raise ValueError("%d tokens fill %d blocks; %d were asked for" % (self.n_tokens, want, n_blocks))
        self.table = self.alloc.allocate(want)
        return list(self.table)

    def internal_waste(self) -> int:
        """Reserved but unwritten slots in the table (below block_size)."""
        return len(self.table) * self.alloc.block_size - self.n_tokens
