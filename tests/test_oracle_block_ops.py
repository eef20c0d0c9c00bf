"""Pins of the block-copy oracle (copy-on-write and swap) -- CPU only.

The copy is pinned through what the pages say it is for: after a branch
copies the shared block it is about to write ([nano-vllm blog §4.3]) and
writes its new token into the copy, the sequence that kept the original
attends exactly as before, and the branch attends as if it had always owned
private blocks holding its tokens -- both checked against torch's
scaled-dot-product attention in float64 on contiguous K/V.  A swap out to CPU
memory and back into other physical blocks ([nano-vllm blog §2.2]) leaves the
attention output unchanged once the table names the new blocks.  Planted
mistakes (half a block, one head, a shifted block) must fail these pins.
"""
import math

import numpy as np
import pytest

import oracle
from tests.test_oracle_pins import random_paged_case, sdpa_dense, oracle_decode


def _branch_case(seed=21, prefix=37, Hkv=2, D=16, bs=16):
    """Sequence A of `prefix` tokens; sequence B shares all of A's blocks (the
    last one only partly filled) and is about to append one token."""
    q, K, V, pool, bt, lens = random_paged_case(seed, [prefix], 4, Hkv, D, bs, spare_blocks=4)
    rng = np.random.default_rng(seed + 1)
    k_new = rng.standard_normal((Hkv, D)).astype(np.float16)
    v_new = rng.standard_normal((Hkv, D)).astype(np.float16)
    q_b = rng.standard_normal((1, 4, D)).astype(np.float16)
    return q, K[0], V[0], pool, bt[0], k_new, v_new, q_b


def _cow_append(copy_fn, seed=21, prefix=37, bs=16):
    q, K, V, pool, row, k_new, v_new, q_b = _branch_case(seed, prefix, bs=bs)
    nb = pool.shape[0]
    used = set(int(x) for x in row)
    fresh = next(b for b in range(nb) if b not in used)
    tail = prefix // bs                       # logical block the new token goes into
    assert prefix % bs != 0                  # the shared tail block is partly filled
    pool_cow = copy_fn(pool, pool, [[int(row[tail]), fresh]])
    row_b = row.copy()
    row_b[tail] = fresh
    L_b = prefix + 1
    bt_b = row_b.reshape(1, -1).astype(np.int32)
    pool_w = oracle.cache_write(pool_cow, "f16", k_new.view(np.uint16)[None], v_new.view(np.uint16)[None], "f16",
                                bt_b, np.array([L_b], dtype=np.int32), bs)
    scale = 1.0 / math.sqrt(K.shape[2])
    out_a = oracle_decode(q, pool_w, row.reshape(1, -1).astype(np.int32), np.array([prefix], dtype=np.int32), bs, scale)
    out_b = oracle_decode(q_b, pool_w, bt_b, np.array([L_b], dtype=np.int32), bs, scale)
    ref_a = sdpa_dense(q, [K], [V], scale)
    ref_b = sdpa_dense(q_b, [np.concatenate([K, k_new[None]])], [np.concatenate([V, v_new[None]])], scale)
    return out_a, ref_a, out_b, ref_b


@pytest.mark.parametrize("prefix,bs", [(37, 16), (20, 16), (70, 32)])
def test_copy_on_write_branch(prefix, bs):
    out_a, ref_a, out_b, ref_b = _cow_append(oracle.copy_blocks, prefix=prefix, bs=bs)
    np.testing.assert_allclose(out_a, ref_a, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out_b, ref_b, rtol=0, atol=1e-12)


def test_write_without_copy_corrupts_the_sharer():
    """Control: appending into the shared block without the copy changes the
    other sequence's output (what copy-on-write exists to prevent)."""
    q, K, V, pool, row, k_new, v_new, _ = _branch_case()
    L_b = 38
    pool_w = oracle.cache_write(pool, "f16", k_new.view(np.uint16)[None], v_new.view(np.uint16)[None], "f16",
                                row.reshape(1, -1).astype(np.int32), np.array([L_b], dtype=np.int32), 16)
    scale = 1.0 / math.sqrt(K.shape[2])
    out_a2 = oracle_decode(q, pool_w, row.reshape(1, -1).astype(np.int32), np.array([L_b], dtype=np.int32), 16, scale)
    assert np.abs(out_a2 - sdpa_dense(q, [K], [V], scale)).max() > 1e-3


def test_swap_out_and_back_into_other_blocks():
    """Swap a sequence's blocks out to a host pool and back into different
    physical blocks: with the table renamed, attention is unchanged."""
    q, K, V, pool, bt, lens = random_paged_case(31, [50, 9], 4, 2, 16, 16, spare_blocks=8)
    scale = 1.0 / 4.0
    before = oracle_decode(q, pool, bt, lens, 16, scale)
    s = 0
    blocks = [int(x) for x in bt[s, :-(-50 // 16)]]
    host = np.zeros((len(blocks),) + pool.shape[1:], dtype=pool.dtype)
    host = oracle.copy_blocks(pool, host, [[b, i] for i, b in enumerate(blocks)])
    in_use = set(int(x) for x in bt.ravel() if x >= 0)
    targets = [b for b in range(pool.shape[0]) if b not in in_use][:len(blocks)]
    cleared = pool.copy()
    cleared[blocks] = np.float16(np.nan).view(np.uint16)      # the old blocks are reused by others
    back = oracle.copy_blocks(host, cleared, [[i, t] for i, t in enumerate(targets)])
    bt2 = bt.copy()
    bt2[s, :len(targets)] = targets
    after = oracle_decode(q, back, bt2, lens, 16, scale)
    np.testing.assert_array_equal(after, before)


def test_mapping_contract_is_checked():
    pool = np.zeros((4, 2, 16, 1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 4]])               # out of range
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 1], [2, 1]])       # destination twice
    with pytest.raises(ValueError):
        oracle.copy_blocks(pool, pool, [[0, 1], [1, 2]])       # chained inside one pool
    other = np.zeros((4, 2, 16, 1, 8), dtype=np.uint16)
    oracle.copy_blocks(pool, other, [[0, 1], [1, 0]])          # swapping between pools is fine


MUTANTS = {
    "k_half_only": lambda out, src, s, d: out.__setitem__((d, 0), src[s, 0]),
    "one_head": lambda out, src, s, d: out.__setitem__((d, slice(None), slice(None), 0), src[s, :, :, 0]),
    "shifted_block": lambda out, src, s, d: out.__setitem__(d, src[(s + 1) % src.shape[0]]),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_copy_mistakes_are_caught(mutant):
    def bad_copy(src_pool, dst_pool, mapping):
        out = dst_pool.copy()
        for s, d in np.asarray(mapping).reshape(-1, 2):
            MUTANTS[mutant](out, src_pool, int(s), int(d))
        return out
    out_a, ref_a, out_b, ref_b = _cow_append(bad_copy)
    assert np.abs(out_b - ref_b).max() > 1e-6 or not np.isfinite(out_b).all()
