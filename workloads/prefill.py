"""Seeded synthetic inputs for the prompt stage: packed new tokens per sequence.

A batch has, per sequence, a final length L_s and a number n_s <= L_s of new
tokens (n_s = L_s for a fresh prompt, fewer when a prefix is already cached,
[nano-vllm blog §4.3]).  The new tokens' queries, keys and values are packed
back to back in sequence order; ``cu_seqlens`` holds the run boundaries
(0, n_0, n_0 + n_1, ...) as in [CANN notes §3.1].

Values are drawn from ``numpy.random.default_rng(seed)`` in a fixed order:
block-table permutation -> pool key half -> pool value half -> packed new
keys -> packed new values -> packed queries; N(0, 1) float32 cast to the
storage dtype with round-to-nearest-even.  The pool is filled slot for slot
(cached prefix slots hold real values; the new tokens' slots hold whatever
the fill put there until the multi-token write overwrites them).  For fp8 KV
the pool and the new K/V are returned as bf16 source values plus per-tensor
scales (max |x| / 448); encoding is the consumer's job.

Nothing here addresses the pool or encodes fp8.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .block_manager import BlockManager, blocks_for_tokens
from .configs import MIXED_LENS, _normal_bits, bf16_bits_to_f32


@dataclass
class PrefillBatch:
    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    src_dtype: str
    scale: float
    k_scale: float
    v_scale: float
    context_lens: np.ndarray     # int32 [B], lengths with the new tokens included
    new_lens: np.ndarray         # int32 [B], n_s
    cu_seqlens: np.ndarray       # int32 [B + 1]
    tables: list
    manager: BlockManager
    max_blocks_per_seq: int
    query: np.ndarray            # raw bits [T, Hq, D] of q_dtype
    new_key: np.ndarray          # raw bits [T, Hkv, D] of src_dtype
    new_value: np.ndarray
    kv_pool: np.ndarray | None   # raw bits [NB, 2, bs, Hkv, D] (16-bit KV)
    kv_source: np.ndarray | None  # bf16 bits (fp8 KV, pre-quantisation)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def block_table_array(self, pad: int = -1) -> np.ndarray:
        out = np.full((self.num_seqs, self.max_blocks_per_seq), pad, dtype=np.int32)
        for s, tab in enumerate(self.tables):
            out[s, :len(tab)] = tab
        return out


def make_prefill(name: str, seed: int, context_lens, new_lens, num_heads: int, num_kv_heads: int,
                 head_dim: int, block_size: int, q_dtype: str, kv_dtype: str, spare: float = 0.10,
                 max_blocks_per_seq: int | None = None) -> PrefillBatch:
    lens = np.asarray(context_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    if lens.shape != new.shape or (new < 0).any() or (new > lens).any():
        raise ValueError("need 0 <= new_lens <= context_lens")
    rng = np.random.default_rng(seed)
    bs = int(block_size)
    used = sum(blocks_for_tokens(int(L), bs) for L in lens)
    num_blocks = max(int(np.ceil(used * (1.0 + spare))), 1)
    manager = BlockManager(num_blocks, bs, rng)
    tables = []
    for L in lens:
        tab: list[int] = []
        manager.grow_to(tab, int(L))
        tables.append(tab)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max([blocks_for_tokens(int(L), bs) for L in lens] + [1])
    Hq, Hkv, D = num_heads, num_kv_heads, head_dim
    src = "bf16" if kv_dtype == "fp8_e4m3" else kv_dtype
    pool = np.empty((num_blocks, 2, bs, Hkv, D), dtype=np.uint16)
    pool[:, 0] = _normal_bits(rng, (num_blocks, bs, Hkv, D), src)
    pool[:, 1] = _normal_bits(rng, (num_blocks, bs, Hkv, D), src)
    T = int(new.sum())
    new_key = _normal_bits(rng, (T, Hkv, D), src)
    new_value = _normal_bits(rng, (T, Hkv, D), src)
    query = _normal_bits(rng, (T, Hq, D), q_dtype)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(new)
    k_scale = v_scale = 1.0
    kv_pool, kv_source = pool, None
    if kv_dtype == "fp8_e4m3":
        k_scale = float(np.float32(max(float(np.abs(bf16_bits_to_f32(pool[:, 0])).max()),
                                       float(np.abs(bf16_bits_to_f32(new_key)).max(initial=0.0))) / 448.0))
        v_scale = float(np.float32(max(float(np.abs(bf16_bits_to_f32(pool[:, 1])).max()),
                                       float(np.abs(bf16_bits_to_f32(new_value)).max(initial=0.0))) / 448.0))
        kv_pool, kv_source = None, pool
    return PrefillBatch(
        name=name, seed=seed, num_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
        q_dtype=q_dtype, kv_dtype=kv_dtype, src_dtype=src, scale=float(np.float32(1.0 / np.sqrt(D))),
        k_scale=k_scale, v_scale=v_scale, context_lens=lens.astype(np.int32), new_lens=new.astype(np.int32),
        cu_seqlens=cu, tables=tables, manager=manager, max_blocks_per_seq=int(max_blocks_per_seq),
        query=query, new_key=new_key, new_value=new_value, kv_pool=kv_pool, kv_source=kv_source)


def make_prefill_mixed(seed: int = 3, block_size: int = 16) -> PrefillBatch:
    """The packed prompt batch of [CANN notes §1.2]: 8 fresh prompts of lengths
    128, 200, 512, 1024, 2048, 256, 64, 1024 (5256 tokens), 32/32 heads,
    head_dim 128, fp16."""
    return make_prefill(f"prefill_mixed_bs{block_size}", seed, MIXED_LENS, MIXED_LENS, 32, 32, 128,
                        block_size, "f16", "f16")
