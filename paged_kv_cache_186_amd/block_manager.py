"""Host-side bookkeeping for the paged KV cache: free list, block tables,
reference counts, slot numbers and copy-on-write plans.

Nothing here touches the GPU.  It decides *where* each token's K/V lives; the
kernels in ``libpagedattn`` only read and write the places it names.

Semantics follow the vLLM tutorial page "3. PagedAttention原理":

* §3.3.2 — a request receives one physical block when it starts; each new
  token goes into the last block while that block has room, and a block is
  taken from the free list only when the last one is full; when a request ends
  all of its physical blocks go back to the free list for immediate reuse.
* §3.3.4 (the teaching class) — the free list starts as every block id in
  increasing order and blocks are taken from its end; running out of blocks is
  an error (``RuntimeError``).
* §3.3.3 and the pitfall note after §3.3.4 — blocks may be shared by several
  requests (common prefixes, beam search); each block keeps a reference count
  and only returns to the free list when the count reaches zero.
* Copy-on-write of a shared block before a private write follows
  "mlx-paged-attention: Bringing vLLM-level High Throughput Inference to Apple
  Silicon", core feature 2, and PagedAttentionMetal's section 块表管理 (the
  table makes copying and sharing of blocks cheap).

A slot number is ``physical_block * block_size + row``; it is what
``pa_reshape_and_cache`` consumes.
"""

from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            self.free: List[int] = list(range(self.num_blocks))
        else:
            self.free = [int(b) for b in free_order]
            if sorted(self.free) != list(range(self.num_blocks)):
                raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.refcount = np.zeros(self.num_blocks, dtype=np.int64)
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- allocation -----------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise RuntimeError("KV block pool exhausted: no free physical block")
        b = self.free.pop()
        self.refcount[b] = 1
        return b

    def num_free(self) -> int:
        return len(self.free)

    def allocate(self, seq_id: int) -> int:
        """Start a request: it owns one (empty) physical block."""
        if seq_id in self.tables:
            raise ValueError(f"sequence {seq_id} already allocated")
        b = self._take()
        self.tables[seq_id] = [b]
        self.lens[seq_id] = 0
        return b

    def make_private(self, seq_id: int, logical_block: int) -> Optional[Tuple[int, int]]:
        """Copy-on-write: give ``seq_id`` its own copy of a shared block.

        Returns the (src, dst) pair the caller must copy on the device
        (``pa_copy_blocks``), or None when the block is already private.
        """
        table = self.tables[seq_id]
        src = table[logical_block]
        if self.refcount[src] <= 1:
            return None
        dst = self._take()
        self.refcount[src] -= 1
        table[logical_block] = dst
        return (src, dst)

    def append_slot(self, seq_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the cache slot of the sequence's next token.

        Returns (slot, cow_pair).  A fresh block is taken exactly when the last
        block is full; if the last block still has room but is shared, it is
        first made private and ``cow_pair`` names the copy to perform.
        """
        table = self.tables[seq_id]
        n = self.lens[seq_id]
        bs = self.block_size
        cow = None
        if n == len(table) * bs:
            table.append(self._take())
        else:
            cow = self.make_private(seq_id, n // bs)
        slot = table[n // bs] * bs + n % bs
        self.lens[seq_id] = n + 1
        return slot, cow

    def append_slots(self, seq_id: int, count: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots, cows = [], []
        for _ in range(count):
            s, c = self.append_slot(seq_id)
            slots.append(s)
            if c is not None:
                cows.append(c)
        return slots, cows

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (refcounts go up)."""
        if child in self.tables:
            raise ValueError(f"sequence {child} already allocated")
        table = list(self.tables[parent])
        for b in table:
            self.refcount[b] += 1
        self.tables[child] = table
        self.lens[child] = self.lens[parent]

    def free_seq(self, seq_id: int) -> None:
        """End a request; blocks whose count reaches zero return to the free list."""
        if seq_id not in self.tables:
            raise KeyError(f"sequence {seq_id} is not allocated")
        for b in self.tables.pop(seq_id):
            if self.refcount[b] <= 0:
                raise RuntimeError(f"reference count underflow on block {b}")
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lens[seq_id]

    # -- views ------------------------------------------------------------------
    def context_len(self, seq_id: int) -> int:
        return self.lens[seq_id]

    def slot_of(self, seq_id: int, position: int) -> int:
        table = self.tables[seq_id]
        if not 0 <= position < self.lens[seq_id]:
            raise IndexError("position outside the sequence")
        return table[position // self.block_size] * self.block_size + position % self.block_size

    def block_tables(self, seq_ids: Iterable[int], width: Optional[int] = None) -> np.ndarray:
        """int32 [S, width] array; entries past a sequence's blocks are -1."""
        seq_ids = list(seq_ids)
        need = [-(-self.lens[s] // self.block_size) for s in seq_ids]
        w = max([1] + need) if width is None else int(width)
        if any(n > w for n in need):
            raise ValueError("width smaller than a sequence's block count")
        out = -np.ones((len(seq_ids), w), dtype=np.int32)
        for i, s in enumerate(seq_ids):
            n = need[i]
            out[i, :n] = self.tables[s][:n]
        return out

    def context_lens(self, seq_ids: Iterable[int]) -> np.ndarray:
        return np.array([self.lens[s] for s in seq_ids], dtype=np.int32)
