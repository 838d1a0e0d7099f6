"""Block ownership model — TEST INFRASTRUCTURE ONLY (part of the oracle).

Only the tests use this module; it shares nothing with the library's allocator.

"KV Cache: capacity, layout, lifecycle" (wineandchord):
- "Lifecycle and ownership": a block is free, exclusive or shared read-only; its
  reference count is the number of sequences that still hold it; a shared block
  is copied before anyone writes into it; each release happens once.
- "Reference counting and tail-block COW": a fork hands the child the parent's
  table and adds one reference to every block in it; the next token of a
  sequence goes to (logical block, offset) = divmod(committed length, B); at
  offset 0 the sequence takes a fresh block, and inside a block that another
  sequence also holds it first moves to a fresh block, dropping one reference to
  the old one.  The free list hands out its last element first.
"03 | PagedAttention and the KV-cache memory system", §5: the free queue and the
reference counts of shared prefix blocks.

Where the pages are silent (the order in which a finished sequence's blocks go
back to the free list) the model takes this reading: the pages hand out the last
element of the free list, and a release pushes the sequence's blocks in reverse
table order, so that the list gives them back in the order the sequence took
them (its first block is handed out next).
"""
from __future__ import annotations


class NoFreeBlock(Exception):
    """A fresh block was needed and the free list is empty (nothing changed)."""


class BlockModel:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.block_size = block_size
        self.refcount = [0] * num_blocks
        # the free list, handed out from its end
        self.free = list(free_order) if free_order is not None else list(range(num_blocks))[::-1]
        self.tables = {}   # live sequence -> list of physical blocks
        self.lengths = {}  # live sequence -> committed tokens
        self._next = 0

    def add_seq(self) -> int:
        sid = self._next
        self._next += 1
        self.tables[sid] = []
        self.lengths[sid] = 0
        return sid

    def fork(self, parent: int) -> int:
        table = self.tables[parent]  # KeyError: unknown or released
        child = self.add_seq()
        self.tables[child] = list(table)
        self.lengths[child] = self.lengths[parent]
        for b in table:
            self.refcount[b] += 1
        return child

    def append(self, sid: int):
        """(slot, (cow_src, cow_dst)) of the sequence's next token, then commit it."""
        table = self.tables[sid]
        logical, offset = divmod(self.lengths[sid], self.block_size)
        cow = (-1, -1)
        if offset == 0:
            if not self.free:
                raise NoFreeBlock()
            fresh = self.free.pop()
            self.refcount[fresh] = 1
            table.append(fresh)
        elif self.refcount[table[logical]] > 1:
            if not self.free:
                raise NoFreeBlock()
            fresh = self.free.pop()
            shared = table[logical]
            self.refcount[shared] -= 1
            self.refcount[fresh] = 1
            table[logical] = fresh
            cow = (shared, fresh)
        self.lengths[sid] += 1
        return table[logical] * self.block_size + offset, cow

    def free_seq(self, sid: int):
        table = self.tables.pop(sid)  # KeyError the second time: one release only
        del self.lengths[sid]
        for b in reversed(table):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
