"""ctypes binding of the host block manager with prefix cache (include/pa_block_manager.h).

Argument marshalling only: every decision (cache walk, reference counts,
LRU eviction, copy-on-write) is made in libpa.so.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._lib import STATUS_NAMES, load


class PoolExhausted(RuntimeError):
    """The manager could not find enough free blocks ("KV cache block pool exhausted")."""


class _Stats(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("free_blocks", ctypes.c_int32),
                ("cached_free_blocks", ctypes.c_int32), ("cached_blocks", ctypes.c_int32),
                ("num_sequences", ctypes.c_int32), ("lookups", ctypes.c_int64), ("hits", ctypes.c_int64),
                ("evictions", ctypes.c_int64)]


def _i32p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class BlockManager:
    """Physical KV blocks, per-sequence block tables and a prefix cache."""

    def __init__(self, num_blocks: int, block_size: int, extra_key: int = 0, initial_order=None):
        self._lib = load()
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_order must hold num_blocks block ids")
        self._h = self._lib.pa_bm_create(int(num_blocks), int(block_size), int(extra_key) & (2**64 - 1),
                                         None if order is None else _i32p(order))
        if not self._h:
            raise ValueError("invalid block manager arguments")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_bm_destroy(h)

    def _check(self, st: int, what: str) -> None:
        if st == 8:
            raise PoolExhausted("KV cache block pool exhausted")
        if st != 0:
            raise RuntimeError(f"{what} failed: {STATUS_NAMES.get(st, st)}")

    def add_sequence(self, seq_id: int, tokens) -> int:
        """Admit a sequence with its prompt; returns the number of leading
        prompt tokens whose KV is already cached (a multiple of block_size)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        cached = ctypes.c_int32(0)
        self._check(self._lib.pa_bm_add_sequence(self._h, int(seq_id), _i32p(toks), int(toks.size),
                                                 ctypes.byref(cached)), "pa_bm_add_sequence")
        return int(cached.value)

    def append_token(self, seq_id: int, token: int) -> None:
        self._check(self._lib.pa_bm_append_token(self._h, int(seq_id), int(token)), "pa_bm_append_token")

    def fork(self, parent_id: int, child_id: int) -> None:
        self._check(self._lib.pa_bm_fork(self._h, int(parent_id), int(child_id)), "pa_bm_fork")

    def free_sequence(self, seq_id: int) -> None:
        self._check(self._lib.pa_bm_free_sequence(self._h, int(seq_id)), "pa_bm_free_sequence")

    def take_copies(self, max_pairs: int = 1 << 16) -> np.ndarray:
        """Queued copy-on-write copies as an int32 [n, 2] array of (source, destination)."""
        buf = np.empty((max_pairs, 2), dtype=np.int32)
        n = self._lib.pa_bm_take_copies(self._h, _i32p(buf), int(max_pairs))
        return buf[:n].copy()

    def sequence_length(self, seq_id: int) -> int:
        return int(self._lib.pa_bm_sequence_length(self._h, int(seq_id)))

    def block_table(self, seq_id: int) -> list[int]:
        n = self._lib.pa_bm_block_table(self._h, int(seq_id), None, 0)
        if n < 0:
            raise KeyError(seq_id)
        buf = np.empty(max(n, 1), dtype=np.int32)
        self._lib.pa_bm_block_table(self._h, int(seq_id), _i32p(buf), n)
        return buf[:n].tolist()

    def block_tables(self, seq_ids, max_blocks: int, pad: int = -1) -> np.ndarray:
        """int32 [len(seq_ids), max_blocks] table array for the kernels."""
        out = np.full((len(seq_ids), max_blocks), pad, dtype=np.int32)
        for r, s in enumerate(seq_ids):
            t = self.block_table(s)
            if len(t) > max_blocks:
                raise ValueError("block table longer than max_blocks")
            out[r, :len(t)] = t
        return out

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_bm_ref_count(self._h, int(block)))

    def stats(self) -> dict:
        st = _Stats()
        self._check(self._lib.pa_bm_stats_get(self._h, ctypes.byref(st)), "pa_bm_stats_get")
        return {name: getattr(st, name) for name, _ in _Stats._fields_}
