"""Float64 CPU oracle: paged decode attention and the per-token KV cache write.

Test infrastructure only (see the package docstring).  Everything here is the
plain definition, written for a reader to check against the pages:

* KV pool layout [num_blocks, 2, block_size, num_kv_heads, head_dim], index 1
  selecting K (0) or V (1) -- [CANN notes §2.1].
* Logical token t of sequence s lives in physical block
  ``block_table[s][t // block_size]`` at in-block offset ``t % block_size``
  -- [CANN notes §2.2]; the table maps logical block -> physical block
  ([nano-vllm blog §2.2]).
* Decode attention walks the sequence's blocks, keeps only the valid tokens of
  the partially filled last block, takes a softmax over the scores and sums V
  with those weights -- [nano-vllm blog §2.3]; the newest token is written
  first and then every block is read -- [CANN notes §4.3].
* The cache write puts the new token's K and V at that same (block, offset)
  -- [nano-vllm blog §4.1 step 3], [CANN notes §4.3 steps 1-3].

Readings where the pages are silent (each one listed with the others in the
design notes): the softmax scale is an argument (the pages apply none); query
head h reads KV head ``h // (num_heads // num_kv_heads)``; a sequence of
length 0 yields a zero output and no write; fp8 values are ``code * scale``.
"""
from __future__ import annotations

import numpy as np

from .fp8_e4m3 import e4m3_decode, e4m3_quantise


def to_f64(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits -> float64 values (exact for all three dtypes)."""
    raw = np.asarray(raw)
    if dtype == "f16":
        return raw.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bfloat16 is the upper half of an IEEE binary32.
        return (raw.view(np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return e4m3_decode(raw.view(np.uint8))
    raise ValueError(f"unknown dtype {dtype}")


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """KV bytes one token costs: 2 (K and V) x layers x KV heads x head_dim x bytes.

    [nano-vllm blog §1.1], [CANN notes §1.1]."""
    return 2 * num_layers * num_kv_heads * head_dim * elem_bytes


def slot_of(block_table_row, t: int, block_size: int) -> tuple[int, int]:
    """(physical block, in-block offset) of logical token t -- [CANN notes §2.2]."""
    return int(block_table_row[t // block_size]), int(t % block_size)


def num_blocks_of(context_len: int, block_size: int) -> int:
    """Blocks a sequence occupies: ceil(len / block_size) -- [CANN notes §2.3, §4.2]."""
    return -(-int(context_len) // int(block_size))


def gather_kv(kv_pool: np.ndarray, kv_dtype: str, block_table_row, context_len: int,
              block_size: int) -> tuple[np.ndarray, np.ndarray]:
    """Contiguous float64 K and V, [L, num_kv_heads, head_dim], of one sequence.

    Only tokens 0..L-1 are read; slots past the valid length of the last block
    are never touched (the tail mask of [nano-vllm blog §2.3])."""
    num_blocks = kv_pool.shape[0]
    L = int(context_len)
    n = num_blocks_of(L, block_size)
    row = np.asarray(block_table_row)
    if n > row.shape[0]:
        raise ValueError("block table shorter than the sequence")
    if n and ((row[:n] < 0).any() or (row[:n] >= num_blocks).any()):
        raise ValueError("block table entry outside the pool")
    t = np.arange(L)
    blk = row[t // block_size]
    off = t % block_size
    K = to_f64(kv_pool[blk, 0, off], kv_dtype)
    V = to_f64(kv_pool[blk, 1, off], kv_dtype)
    return K, V


def paged_decode(query: np.ndarray, q_dtype: str, kv_pool: np.ndarray, kv_dtype: str,
                 block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                 scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                 seqs=None) -> np.ndarray:
    """Decode attention output, float64 [B, num_heads, head_dim].

    For each sequence: gather its K/V through the block table, then for each
    query head h with KV head g = h // (num_heads / num_kv_heads):
        z_t = scale * <q_h, K_t,g>         (times k_scale for fp8 KV)
        p   = softmax(z)                   (textbook: exp(z - max z) / sum)
        out = sum_t p_t * V_t,g            (times v_scale for fp8 KV)
    ``seqs`` restricts the work to a subset of sequences (other rows stay 0).
    """
    q = to_f64(query, q_dtype)
    B, Hq, D = q.shape
    NB, two, bs, Hkv, D2 = kv_pool.shape
    if two != 2 or bs != block_size or D2 != D or Hq % Hkv:
        raise ValueError("shape mismatch between query and KV pool")
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for s in (range(B) if seqs is None else seqs):
        L = int(context_lens[s])
        if L <= 0:
            continue
        K, V = gather_kv(kv_pool, kv_dtype, block_tables[s], L, block_size)
        if kv_dtype == "fp8_e4m3":
            K = K * float(k_scale)
            V = V * float(v_scale)
        for h in range(Hq):
            g = h // group
            z = float(scale) * (K[:, g, :] @ q[s, h])
            e = np.exp(z - z.max())
            p = e / e.sum()
            out[s, h] = p @ V[:, g, :]
    return out


def encode_for_cache(x_raw: np.ndarray, src_dtype: str, kv_dtype: str, scale: float) -> np.ndarray:
    """Values as stored in the pool: a bit copy for 16-bit KV, e4m3 codes for fp8."""
    if kv_dtype == src_dtype:
        return np.array(x_raw, copy=True)
    if kv_dtype == "fp8_e4m3" and src_dtype in ("bf16", "f16"):
        x32 = to_f64(x_raw, src_dtype).astype(np.float32)     # exact widening
        return e4m3_quantise(x32, scale)
    raise ValueError(f"unsupported write {src_dtype} -> {kv_dtype}")


def cache_write(kv_pool: np.ndarray, kv_dtype: str, key: np.ndarray, value: np.ndarray,
                src_dtype: str, block_tables: np.ndarray, context_lens: np.ndarray,
                block_size: int, k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """Pool after writing each sequence's newest token (t = len - 1).

    ``context_lens`` are the lengths *after* the append; a length <= 0 writes
    nothing.  Returns a new array; the input pool is not modified."""
    pool = np.array(kv_pool, copy=True)
    B = key.shape[0]
    for s in range(B):
        L = int(context_lens[s])
        if L <= 0:
            continue
        b, o = slot_of(block_tables[s], L - 1, block_size)
        if not 0 <= b < pool.shape[0]:
            raise ValueError("block table entry outside the pool")
        pool[b, 0, o] = encode_for_cache(key[s], src_dtype, kv_dtype, k_scale)
        pool[b, 1, o] = encode_for_cache(value[s], src_dtype, kv_dtype, v_scale)
    return pool


def encode_pool(source_raw: np.ndarray, src_dtype: str, kv_dtype: str,
                k_scale: float, v_scale: float) -> np.ndarray:
    """Encode a whole pool of source values slot by slot (K half with k_scale, V half with v_scale)."""
    out = np.empty(source_raw.shape, dtype=np.uint8 if kv_dtype == "fp8_e4m3" else source_raw.dtype)
    out[:, 0] = encode_for_cache(source_raw[:, 0], src_dtype, kv_dtype, k_scale)
    out[:, 1] = encode_for_cache(source_raw[:, 1], src_dtype, kv_dtype, v_scale)
    return out
