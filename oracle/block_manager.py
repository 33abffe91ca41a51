"""Plain model of fixed-size KV block accounting.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows [PA] ("What is PagedAttention?"):
* block-table section: KV is kept in blocks of a fixed number of tokens; each
  request has its own table of physical blocks in logical order; the current
  block is filled while it has room and a block is added when it is full; the
  unused tail of the last block is the only waste;
* "Reusing blocks freed when a request ends": a finished request returns its
  blocks, any request may take them, they need not be adjacent to anything, and
  nothing is compacted;
* "Sharing common blocks and copy-on-write": several sequences may point at
  the same physical block; a reference count keeps it alive until no sequence
  uses it; before a sequence writes into a shared block it gets its own copy and
  its table is repointed;
* the limits section: when the pool has no free block the request must wait
  (modelled as an exception).
"""
from __future__ import annotations

from collections import deque


class PoolExhausted(RuntimeError):
    """No free block is left; the caller has to wait for one to be released."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else list(free_order)
        self.free = deque(order)
        self.refcount = {b: 0 for b in order}
        self.tables: dict = {}
        self.lengths: dict = {}
        self.copies: list = []            # (src, dst) block copies made by copy-on-write

    # -- helpers ------------------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise PoolExhausted("no free KV block")
        b = self.free.popleft()
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    # -- requests -----------------------------------------------------------------
    def add(self, seq, n_tokens: int = 0) -> None:
        """A new request with ``n_tokens`` already to store."""
        self.tables[seq] = []
        self.lengths[seq] = 0
        self.append(seq, n_tokens)

    def append(self, seq, n_tokens: int = 1) -> None:
        """Store ``n_tokens`` more tokens of ``seq`` one at a time: a full (or
        missing) last block means a new block; a shared last block with room is
        copied first (copy-on-write)."""
        table = self.tables[seq]
        for _ in range(n_tokens):
            used = self.lengths[seq] - (len(table) - 1) * self.block_size if table else self.block_size
            if used == self.block_size:
                table.append(self._take())
            elif self.refcount[table[-1]] > 1:
                dst = self._take()
                self.copies.append((table[-1], dst))
                self._release(table[-1])
                table[-1] = dst
            self.lengths[seq] += 1

    def fork(self, parent, child) -> None:
        """``child`` starts with ``parent``'s tokens and shares its blocks."""
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def finish(self, seq) -> None:
        """The request ends; blocks no other sequence uses become free."""
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lengths[seq]

    # -- accounting ---------------------------------------------------------------
    def num_blocks(self, seq) -> int:
        return len(self.tables[seq])

    def spare_slots(self, seq) -> int:
        return len(self.tables[seq]) * self.block_size - self.lengths[seq]

    def num_free(self) -> int:
        return len(self.free)
