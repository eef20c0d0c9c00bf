"""Host-side allocator of physical KV blocks: a free list plus reference counts.

Follows the allocator the pages describe:
  * [nano-vllm blog §2.2]: a flat pool of ``num_blocks`` equal blocks, a free
    list, ``allocate(n)`` that raises "KV cache block pool exhausted" when the
    list is short, and ``free`` that returns blocks; a new block is taken only
    once the tail block is full.
  * [CANN notes §2.3]: ``ceil(prompt_len / block_size)`` blocks at prompt
    time, one more block per decode append when the tail fills, all blocks
    returned when the sequence ends.
  * [vLLM notes, "引用计数与 LRU" / "块级共享"]: a block may be referenced by
    several block tables; it goes back to the free list when its count drops
    to zero.

The free list starts as a seeded permutation of the block ids, so logical
blocks land on scattered physical blocks (the [nano-vllm blog §2.2] point that
blocks come back "in any order").  Which physical block an allocator returns
is not fixed by the pages; outputs must not depend on it.
"""
from __future__ import annotations

from collections import deque

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when an allocation asks for more blocks than the free list holds."""


def blocks_for_tokens(num_tokens: int, block_size: int) -> int:
    """Blocks a sequence of ``num_tokens`` occupies: ceil(num_tokens / block_size)."""
    return -(-int(num_tokens) // int(block_size))


def full_blocks(num_tokens: int, block_size: int) -> int:
    """Blocks completely filled by ``num_tokens`` tokens (only these are shareable
    prefix blocks, [vLLM notes, "边界条件"]: 100 tokens -> 6 full blocks of 16)."""
    return int(num_tokens) // int(block_size)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, rng: np.random.Generator | None = None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = rng.permutation(self.num_blocks) if rng is not None else np.arange(self.num_blocks)
        # free blocks in the order they are handed out; freed blocks queue at the back
        self._free: deque[int] = deque(int(b) for b in order)
        self.ref_count = np.zeros(self.num_blocks, dtype=np.int64)

    # -- allocation ---------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self, n: int) -> list[int]:
        """Take n blocks from the head of the free queue, each with one reference."""
        n = int(n)
        if n < 0:
            raise ValueError("cannot allocate a negative number of blocks")
        if n > len(self._free):
            raise PoolExhausted("KV cache block pool exhausted")
        taken = [self._free.popleft() for _ in range(n)]
        ids = np.asarray(taken, dtype=np.int64)
        if np.any(self.ref_count[ids] != 0):
            raise AssertionError("a block on the free queue still has references")
        self.ref_count[ids] = 1
        return taken

    def share(self, blocks: list[int]) -> list[int]:
        """Attach already-allocated blocks to one more table (refcount + 1)."""
        for b in blocks:
            if self.ref_count[b] <= 0:
                raise ValueError(f"block {b} is not allocated and cannot be shared")
            self.ref_count[b] += 1
        return list(blocks)

    def free(self, blocks: list[int]) -> None:
        """Drop one reference to each block; blocks reaching zero go back to the free list."""
        for b in blocks:
            if self.ref_count[b] <= 0:
                raise ValueError(f"double free of block {b}")
            self.ref_count[b] -= 1
            if self.ref_count[b] == 0:
                self._free.append(int(b))

    # -- sequence helpers ---------------------------------------------------
    def allocate_for_prompt(self, prompt_len: int) -> list[int]:
        return self.allocate(blocks_for_tokens(prompt_len, self.block_size))

    def grow_to(self, table: list[int], new_len: int) -> list[int]:
        """Append blocks to ``table`` until it holds ``new_len`` tokens.

        A new block is taken only when the current tail block is full; returns
        the blocks added (empty when the tail still has room)."""
        added: list[int] = []
        while len(table) * self.block_size < new_len:
            b = self.allocate(1)[0]
            table.append(b)
            added.append(b)
        return added

    def writable(self, block: int) -> bool:
        """A block may be written only while exactly one table references it."""
        return self.ref_count[block] == 1

    def usage(self, tables: list[list[int]], lens) -> dict:
        """Allocation counters of [CANN notes §5.4] and the internal
        fragmentation of [nano-vllm blog §5.1] / [CANN notes §5.1]:

          pool_blocks            blocks in the pool
          allocated_blocks       blocks taken from the free list
          used_blocks            distinct blocks holding at least one token
          block_utilisation      used_blocks / allocated_blocks
          slot_utilisation       tokens / (table blocks x block_size), per table
          waste_tokens_per_seq   mean empty slots in a sequence's blocks (its
                                 last block only; about block_size / 2)
          mean_table_length      mean blocks per table"""
        lens = [int(x) for x in lens]
        used = set()
        slots = 0
        for tab, L in zip(tables, lens):
            n = blocks_for_tokens(L, self.block_size)
            used.update(int(b) for b in tab[:n])
            slots += len(tab) * self.block_size
        allocated = self.num_blocks - self.num_free
        tokens = sum(lens)
        return {
            "pool_blocks": self.num_blocks,
            "allocated_blocks": allocated,
            "used_blocks": len(used),
            "block_utilisation": len(used) / allocated if allocated else 0.0,
            "slot_utilisation": tokens / slots if slots else 0.0,
            "waste_tokens_per_seq": (slots - tokens) / len(lens) if lens else 0.0,
            "mean_table_length": float(np.mean([len(t) for t in tables])) if tables else 0.0,
        }

    def dump(self, tables: list[list[int]], lens: list[int]) -> str:
        """Debug view: each sequence's table with the refcount of every block."""
        lines = [f"free={self.num_free}/{self.num_blocks}"]
        for s, (tab, n) in enumerate(zip(tables, lens)):
            cells = " ".join(f"{b}(rc{int(self.ref_count[b])})" for b in tab)
            lines.append(f"seq {s} len={n}: {cells}")
        return "\n".join(lines)
