"""Float64 CPU oracle: packed (varlen) multi-token KV write and causal prefill
attention over the paged pool.

Test infrastructure only (see the package docstring).

* Packed layout: the new tokens of all sequences sit back to back in one
  array; ``cu_seqlens`` (length num_seqs + 1, starting at 0) marks where each
  sequence's run begins and ends -- [CANN notes §3.1].
* Inside one sequence a query sees only keys at positions not after its own;
  across sequences nothing is visible (a block-diagonal causal mask) --
  [CANN notes §3.1] and [CANN notes §3.2].
* The packed position of a token gives its sequence, and the block table
  gives where its K/V live in the pool -- [CANN notes §3.3].
* In the prompt stage the new K/V are written into the blocks at their
  in-block offsets, the last block only up to the tokens it holds --
  [CANN notes §4.2]; a prompt whose prefix was found in the prefix cache
  only computes and writes its uncached tail, reusing the cached blocks --
  [nano-vllm blog §4.3].

Readings where the pages are silent (listed with the others in the design
notes): ``context_lens[s]`` is the sequence's length after the new tokens are
in place, so its n_s = cu_seqlens[s+1] - cu_seqlens[s] new tokens hold
positions L_s - n_s .. L_s - 1 (n_s = L_s for a prompt with no cached
prefix); the query at position p attends to every token at positions 0..p of
its own sequence, cached prefix included; the softmax scale, fp8 scales and
the query-head to KV-head rule are those of the decode oracle.
"""
from __future__ import annotations

import numpy as np

from .paged_attention import encode_for_cache, gather_kv, slot_of, to_f64


def packed_positions(cu_seqlens, context_lens) -> tuple[np.ndarray, np.ndarray]:
    """(sequence id, position in its sequence) of every packed token."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    total = int(cu[-1])
    seq = np.empty(total, dtype=np.int64)
    pos = np.empty(total, dtype=np.int64)
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        if n > lens[s]:
            raise ValueError("more new tokens than the sequence holds")
        for i in range(n):
            seq[cu[s] + i] = s
            pos[cu[s] + i] = lens[s] - n + i
    return seq, pos


def cache_write_tokens(kv_pool: np.ndarray, kv_dtype: str, key: np.ndarray, value: np.ndarray,
                       src_dtype: str, block_tables: np.ndarray, context_lens, cu_seqlens,
                       block_size: int, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Pool after writing every packed new token's K and V at its slot.

    key, value: raw [total_new_tokens, num_kv_heads, head_dim] of src_dtype."""
    out = kv_pool.copy()
    seq, pos = packed_positions(cu_seqlens, context_lens)
    for j in range(len(seq)):
        blk, off = slot_of(block_tables[seq[j]], int(pos[j]), block_size)
        out[blk, 0, off] = encode_for_cache(key[j], src_dtype, kv_dtype, k_scale)
        out[blk, 1, off] = encode_for_cache(value[j], src_dtype, kv_dtype, v_scale)
    return out


def paged_prefill(query: np.ndarray, q_dtype: str, kv_pool: np.ndarray, kv_dtype: str,
                  block_tables: np.ndarray, context_lens, cu_seqlens, block_size: int,
                  scale: float, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Causal attention of every packed new query over its own sequence.

    query: raw [total_new_tokens, num_heads, head_dim]; returns float64 of the
    same shape.  The pool must already hold every token (new ones included)."""
    total, Hq, D = query.shape
    Hkv = kv_pool.shape[3]
    if kv_pool.shape[2] != block_size or kv_pool.shape[4] != D or Hq % Hkv:
        raise ValueError("shape mismatch between query and KV pool")
    group = Hq // Hkv
    q = to_f64(query, q_dtype)
    out = np.zeros((total, Hq, D))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.asarray(context_lens, dtype=np.int64)
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        if n == 0:
            continue
        L = int(lens[s])
        K, V = gather_kv(kv_pool, kv_dtype, block_tables[s], L, block_size)
        if kv_dtype == "fp8_e4m3":
            K = K * float(k_scale)
            V = V * float(v_scale)
        for i in range(n):
            p = L - n + i                      # this query's position
            j = int(cu[s]) + i
            for h in range(Hq):
                g = h // group
                z = scale * (K[: p + 1, g, :] @ q[j, h])
                w = np.exp(z - z.max())
                out[j, h] = (w / w.sum()) @ V[: p + 1, g, :]
    return out
