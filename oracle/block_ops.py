"""CPU oracle for whole-block KV operations: copy-on-write and swap.

Test infrastructure only (see the package docstring).

* Sequences that share a prefix share its physical blocks; before one of them
  writes into a shared block (a beam or sample branching off), that block is
  copied to a fresh one and only the writer's table is pointed at the copy --
  copy-on-write, [nano-vllm blog §2.2] and [nano-vllm blog §4.3].
* A preempted request's blocks are copied out to CPU memory and copied back
  when it is scheduled again -- [nano-vllm blog §2.2], and the swapped queue
  of [nano-vllm blog §4.2].

Both are the same operation on whole blocks: destination block d gets the
bytes of source block s, K half and V half, every head.  Reading where the
pages are silent: a call takes a list of (source block, destination block)
pairs; no destination block appears twice, and, within one pool, no block is
both a source and a destination, so the order of the pairs does not matter.
"""
from __future__ import annotations

import numpy as np


def check_block_mapping(mapping: np.ndarray, src_num_blocks: int, dst_num_blocks: int,
                        same_pool: bool) -> None:
    """Raise unless every pair is in range and the pairs are independent."""
    mapping = np.asarray(mapping).reshape(-1, 2)
    src, dst = mapping[:, 0], mapping[:, 1]
    if ((src < 0) | (src >= src_num_blocks)).any() or ((dst < 0) | (dst >= dst_num_blocks)).any():
        raise ValueError("block id out of range")
    if len(set(dst.tolist())) != len(dst):
        raise ValueError("a destination block appears twice")
    if same_pool and set(src.tolist()) & set(dst.tolist()):
        raise ValueError("a block is both source and destination")


def copy_blocks(src_pool: np.ndarray, dst_pool: np.ndarray, mapping) -> np.ndarray:
    """dst_pool after copying src_pool[s] -> dst_pool[d] for every pair (s, d).

    Pools are raw arrays [num_blocks, 2, block_size, num_kv_heads, head_dim]
    of any element type; the bytes are copied unchanged.  Pass the same array
    as both pools for a copy inside one pool."""
    if src_pool.shape[1:] != dst_pool.shape[1:] or src_pool.dtype != dst_pool.dtype:
        raise ValueError("pools must have the same block geometry and element type")
    mapping = np.asarray(mapping, dtype=np.int64).reshape(-1, 2)
    check_block_mapping(mapping, src_pool.shape[0], dst_pool.shape[0], src_pool is dst_pool)
    out = dst_pool.copy()
    for s, d in mapping:
        out[d] = src_pool[s]
    return out
