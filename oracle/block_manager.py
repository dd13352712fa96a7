"""Host block manager for a paged KV cache (oracle; test infrastructure only).

Written from the serving-stack page (chenxutan.com), section 2.2 (分页思想)
and section 2.3 (手写一个 Block Manager):

* the cache is cut into fixed-size blocks of ``block_size`` tokens; every
  sequence owns a block table (logical block i -> physical block id), and a
  KV read goes through that table once;
* every physical block carries a reference count so that blocks can be
  shared (fork) and copied on write (CoW);
* ``allocate`` takes a block off the free list and returns None when the
  pool is exhausted (the page's trigger for preemption); the page's free
  list is a Python list popped from its end, and freed blocks are appended
  to that end;
* ``cow`` keeps a block whose count is 1 and otherwise takes a private copy
  and drops one reference to the shared block; with no free block it raises
  MemoryError;
* a sequence appending a token opens a new block when its length is a
  multiple of ``block_size`` and otherwise copies its (possibly shared) tail
  block on write first;
* ``fork`` shares every block of the parent (one more reference each).

Copies must not chain.  Every recorded (src, dst) pair is a copy that has not
run yet, and the block-copy call runs a batch of pairs concurrently.  Forking
while pairs are queued could make the tail block a queued copy's dst shared
again.  The next append would then queue a copy *from* that dst (a chain),
and the parent's freshly stored token would be copied before it lands.
Releasing while pairs are queued can free a queued pair's block and hand it
out again.  So ``fork`` and ``release`` refuse (RuntimeError) while pairs
are queued: the caller takes them, runs them and the stores of the slots
handed out so far, and then forks or releases.

Unlike the page's version, blocks hold no token lists: the data lives in the
device cache, so ``cow`` records the (src, dst) pair that a block-copy call
must carry out, and ``append_slot`` returns the slot (physical block *
block_size + offset) where the new token's K/V is to be stored.
"""
from __future__ import annotations

from typing import List, Optional, Sequence as Seq, Tuple


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Seq[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.ref_count: List[int] = [0] * self.num_blocks
        if free_order is None:
            free_order = range(self.num_blocks)
        self.free_ids: List[int] = [int(b) for b in free_order]
        if sorted(self.free_ids) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.pending_copies: List[Tuple[int, int]] = []

    # -- basic allocation -------------------------------------------------
    def allocate(self) -> Optional[int]:
        if not self.free_ids:
            return None
        bid = self.free_ids.pop()
        self.ref_count[bid] = 1
        return bid

    def incref(self, bid: int) -> None:
        if self.ref_count[bid] <= 0:
            raise ValueError(f"incref of free block {bid}")
        self.ref_count[bid] += 1

    def free(self, bid: int) -> None:
        if self.ref_count[bid] <= 0:
            raise ValueError(f"double free of block {bid}")
        self.ref_count[bid] -= 1
        if self.ref_count[bid] == 0:
            self.free_ids.append(bid)

    # -- copy on write ----------------------------------------------------
    def cow(self, bid: int) -> int:
        if self.ref_count[bid] == 1:
            return bid
        new = self.allocate()
        if new is None:
            raise MemoryError("no free block for copy-on-write")
        self.pending_copies.append((bid, new))
        self.free(bid)
        return new

    def take_copies(self) -> List[Tuple[int, int]]:
        """(src, dst) block pairs recorded since the last call, in CoW order."""
        out, self.pending_copies = self.pending_copies, []
        return out

    @property
    def usage(self) -> float:
        return (self.num_blocks - len(self.free_ids)) / self.num_blocks

    @property
    def used_blocks(self) -> int:
        return self.num_blocks - len(self.free_ids)


class Sequence:
    """One request's logical view: a block table and a token count."""

    def __init__(self, mgr: BlockManager, seq_id: int):
        self.mgr = mgr
        self.seq_id = seq_id
        self.block_table: List[int] = []
        self.length = 0

    def append_slot(self) -> int:
        """Reserve room for one more token; returns its slot."""
        B = self.mgr.block_size
        if self.length % B == 0:
            bid = self.mgr.allocate()
            if bid is None:
                raise MemoryError(f"sequence {self.seq_id}: no free block")
            self.block_table.append(bid)
        else:
            self.block_table[-1] = self.mgr.cow(self.block_table[-1])
        slot = self.block_table[-1] * B + self.length % B
        self.length += 1
        return slot

    def append_slots(self, n: int) -> List[int]:
        return [self.append_slot() for _ in range(n)]

    def fork(self, new_id: int) -> "Sequence":
        if self.mgr.pending_copies:
            raise RuntimeError("fork while copy pairs are queued: take and run them first")
        child = Sequence(self.mgr, new_id)
        child.block_table = list(self.block_table)
        child.length = self.length
        for bid in child.block_table:
            self.mgr.incref(bid)
        return child

    def release(self) -> None:
        if self.mgr.pending_copies:
            raise RuntimeError("release while copy pairs are queued: take and run them first")
        for bid in self.block_table:
            self.mgr.free(bid)
        self.block_table = []
        self.length = 0
